"""mx_block_mse_noalloc (the block error without a workspace, for callers that
cannot allocate) against mx_block_mse through the C ABI, on two calls in a
row whose second tensor is smaller, in both dtypes, and with each output
alone: per-block MSE bit for bit; tensor sums bit for bit where the
workspace call's grid fits the fixed scratch (at most 2048 workgroups),
else within a relative 1e-6 (the no-alloc launch caps its grid, so its
partial sums fall on other workgroups). Nothing here allocates between the
calls it compares except the test's own output tensors."""
import os
import sys

import numpy as np
import pytest
import torch

import microscaling_fp4_block_mx_amd as mx
import oracle
import workloads

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()
    yield
    torch.cuda.synchronize()


def _ok(st):
    assert st == mx.MX_OK, mx.mx_status_string(st) + " " + mx.mx_last_error_detail()


def _with_workspace(x, c, s, bm, sums, stream):
    R, K = x.shape
    wsb = mx.mx_block_mse_workspace_size(R, K)
    ws = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    _ok(mx.mx_block_mse(x.data_ptr(), mx._DTYPES[x.dtype], c.data_ptr(), s.data_ptr(), R, K,
                        bm.data_ptr() if bm is not None else None,
                        sums.data_ptr() if sums is not None else None, ws.data_ptr(), wsb,
                        stream))
    torch.cuda.synchronize()


def _noalloc(x, c, s, bm, sums, stream):
    R, K = x.shape
    _ok(mx.mx_block_mse_noalloc(x.data_ptr(), mx._DTYPES[x.dtype], c.data_ptr(), s.data_ptr(),
                                R, K, bm.data_ptr() if bm is not None else None,
                                sums.data_ptr() if sums is not None else None, stream))


def _case(shape, seed, dtype):
    x = workloads.bf16_laplace_sparse_outliers(seed, shape=shape).cuda()
    if dtype == torch.float32:
        x = x.float()
    c, s = mx.quantize(x, "oas_nf")
    return x, c, s


def test_noalloc_matches_workspace_call_twice_shrinking():
    stream = torch.cuda.current_stream().cuda_stream
    for dtype in (torch.bfloat16, torch.float32):
        # the second call is smaller: fewer workgroups, fewer partial sums;
        # its result must not see the first call's leftovers
        for shape, seed in (((4096, 8192), 81), ((96, 256), 82)):
            say(f"{dtype} {shape}")
            x, c, s = _case(shape, seed, dtype)
            R, K = shape
            want_bm = torch.empty((R, K // 32), dtype=torch.float32, device="cuda")
            want_sums = torch.empty(2, dtype=torch.float64, device="cuda")
            _with_workspace(x, c, s, want_bm, want_sums, stream)
            got_bm = torch.full_like(want_bm, float("nan"))
            got_sums = torch.full_like(want_sums, float("nan"))
            _noalloc(x, c, s, got_bm, got_sums, stream)
            torch.cuda.synchronize()
            assert torch.equal(got_bm.view(torch.int32), want_bm.view(torch.int32))
            if R * K <= 2048 * 1024 * 8:  # the workspace call's grid fits the scratch
                assert torch.equal(got_sums.view(torch.int64), want_sums.view(torch.int64)), \
                    (got_sums.tolist(), want_sums.tolist())
            else:
                for g, w in zip(got_sums.tolist(), want_sums.tolist()):
                    assert abs(g - w) <= 1e-6 * abs(w), (g, w)


def test_noalloc_each_output_alone_and_against_oracle():
    stream = torch.cuda.current_stream().cuda_stream
    x, c, s = _case((512, 4096), 83, torch.bfloat16)
    R, K = x.shape
    sums = torch.empty(2, dtype=torch.float64, device="cuda")
    _noalloc(x, c, s, None, sums, stream)
    bm = torch.empty((R, K // 32), dtype=torch.float32, device="cuda")
    _noalloc(x, c, s, bm, None, stream)
    torch.cuda.synchronize()
    oracle.build(force=not os.path.exists(os.path.join(os.path.dirname(oracle.__file__),
                                                       "libmxref.so")))
    wbm, wsse, wssq = oracle.block_mse(workloads.to_bf16_bits(x), c.cpu().numpy(),
                                       s.cpu().numpy(), threads=8, with_energy=True)
    np.testing.assert_allclose(bm.cpu().numpy(), wbm, rtol=1e-6, atol=0)
    sse, ssq = sums.tolist()
    assert abs(sse - wsse) <= 1e-6 * wsse and abs(ssq - wssq) <= 1e-6 * wssq


def test_noalloc_empty_tensor_writes_zero_sums():
    stream = torch.cuda.current_stream().cuda_stream
    sums = torch.full((2,), 7.0, dtype=torch.float64, device="cuda")
    _ok(mx.mx_block_mse_noalloc(None, mx.MX_BF16, None, None, 0, 64, None, sums.data_ptr(),
                                stream))
    torch.cuda.synchronize()
    assert sums.tolist() == [0.0, 0.0]


def test_noalloc_on_a_side_stream():
    """The scratch address is looked up for the stream's device; work runs on
    that stream."""
    x, c, s = _case((1024, 4096), 84, torch.bfloat16)
    R, K = x.shape
    want_bm = torch.empty((R, K // 32), dtype=torch.float32, device="cuda")
    want_sums = torch.empty(2, dtype=torch.float64, device="cuda")
    _with_workspace(x, c, s, want_bm, want_sums, torch.cuda.current_stream().cuda_stream)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got_bm = torch.empty_like(want_bm)
    got_sums = torch.empty_like(want_sums)
    torch.cuda.synchronize()
    _noalloc(x, c, s, got_bm, got_sums, side.cuda_stream)
    side.synchronize()
    assert torch.equal(got_bm.view(torch.int32), want_bm.view(torch.int32))
    assert torch.equal(got_sums.view(torch.int64), want_sums.view(torch.int64))  # 512 workgroups
