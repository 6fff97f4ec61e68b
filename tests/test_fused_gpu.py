"""GPU parity of mx_quantize_fused (one pass: codes, scales, y, block MSE,
tensor sums) with the separate calls and with the oracle: codes, scales, y
and block MSE bit for bit, tensor sums to a relative 1e-6, in every scale
mode, both dtypes, ragged shapes, with each optional output on or off."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
import microscaling_fp4_block_mx_amd as mx
from test_parity_gpu import THREADS, assert_same_bits, host_view, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()
    oracle.build(force=not os.path.exists(os.path.join(os.path.dirname(oracle.__file__),
                                                       "libmxref.so")))
    yield
    torch.cuda.synchronize()


def same_sum(got: float, want: float) -> bool:
    """Tensor sums agree: both NaN, equal (infinities included), or within a
    relative 1e-6."""
    if np.isnan(want) or np.isnan(got):
        return bool(np.isnan(want) and np.isnan(got))
    return got == want or abs(got - want) <= 1e-6 * abs(want)


def check_fused(x: torch.Tensor, mode: str, label: str):
    xd = x.cuda()
    say(f"{label} fused {mode} {tuple(x.shape)} {x.dtype}")
    c, s, y, bm, sums = mx.quantize_fused(xd, mode)
    c1, s1 = mx.quantize(xd, mode)
    y1 = mx.dequantize(c1, s1, xd.dtype)
    bm1, sums1 = mx.block_mse(xd, c1, s1)
    assert torch.equal(c, c1) and torch.equal(s, s1), f"{label}: codes/scales differ from quantize"
    assert torch.equal(y.view(torch.uint8), y1.view(torch.uint8)), f"{label}: y differs"
    assert torch.equal(bm.view(torch.int32), bm1.view(torch.int32)), f"{label}: block MSE differs"
    a, b = sums.tolist(), sums1.tolist()
    for u, v in zip(a, b):
        assert same_sum(u, v), f"{label}: sums {a} vs {b}"
    # and the oracle
    xh = host_view(x)
    wc, ws = oracle.quantize(xh, mode)
    assert_same_bits(c, wc, f"{label} codes")
    assert_same_bits(s, ws, f"{label} scales")
    assert_same_bits(y, oracle.fakequant(xh, mode), f"{label} y")
    wbm, wsse, wssq = oracle.block_mse(xh, wc, ws, with_energy=True)
    assert np.allclose(bm.cpu().numpy(), wbm, rtol=1e-6, atol=0, equal_nan=True)
    for got, want in zip(a, (wsse, wssq)):
        assert same_sum(got, want), f"{label}: sums {a} vs oracle {(wsse, wssq)}"


@pytest.mark.parametrize("mode", mx.MODES)
def test_fused_ragged(mode):
    rng = np.random.default_rng(61 + mx.MODES.index(mode))
    for rows, k in ((1, 32), (3, 96), (257, 160), (1000, 4096), (4099, 64)):
        x = rng.standard_t(3, (rows, k)) * np.exp(rng.normal(0, 2, (rows, k // 32))).repeat(32, 1)
        xt = torch.from_numpy(x.astype(np.float32))
        check_fused(xt, mode, f"f32 {rows}x{k}")
        check_fused(xt.to(torch.bfloat16), mode, f"bf16 {rows}x{k}")


def test_fused_bench_tensor_and_fp32_config():
    check_fused(workloads.bf16_student_t_outlier_channels(2), "oas", "student-t 8192x4096")
    check_fused(workloads.fp32_normal(1), "ocp", "fp32 normal 1024x4096")


def test_fused_optional_outputs():
    x = workloads.bf16_student_t_outlier_channels(62, shape=(512, 4096)).cuda()
    c, s, y, bm, sums = mx.quantize_fused(x, "ocp")
    for wy, wb, wsum in ((False, False, False), (True, False, False), (False, True, False),
                         (False, False, True), (False, True, True)):
        c2, s2, y2, bm2, sums2 = mx.quantize_fused(x, "ocp", wy, wb, wsum)
        assert torch.equal(c2, c) and torch.equal(s2, s)
        assert (y2 is None) != wy and (bm2 is None) != wb and (sums2 is None) != wsum
        if wy:
            assert torch.equal(y2.view(torch.int16), y.view(torch.int16))
        if wb:
            assert torch.equal(bm2.view(torch.int32), bm.view(torch.int32))
        if wsum:
            assert torch.equal(sums2.view(torch.int64), sums.view(torch.int64))
    # empty tensor: sums written as zeros
    _, _, _, _, z = mx.quantize_fused(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"))
    assert z.tolist() == [0.0, 0.0]


def test_fused_past_2_31_elements():
    """One bf16 tensor of 2^31 + 2^20 elements in OAS mode: every output
    against the separate calls in full, and against the oracle on sampled
    rows including the last ones (64-bit indexing in the one-pass kernel)."""
    rows, k = (1 << 31) // 4096 + 256, 4096
    say(f"fused big tensor [{rows}, {k}]")
    g = torch.Generator(device="cuda")
    g.manual_seed(93)
    x = torch.empty((rows, k), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, rows, 65536):
        r1 = min(rows, r0 + 65536)
        x[r0:r1] = (torch.randn((r1 - r0, k), generator=g, device="cuda") * 3).to(torch.bfloat16)
    c, s, y, bm, sums = mx.quantize_fused(x, "oas")
    c1, s1 = mx.quantize(x, "oas")
    assert torch.equal(c, c1) and torch.equal(s, s1)
    del c1, s1
    y1 = mx.dequantize(c, s, torch.bfloat16)
    assert torch.equal(y.view(torch.int16), y1.view(torch.int16))
    del y1
    bm1, sums1 = mx.block_mse(x, c, s)
    assert torch.equal(bm.view(torch.int32), bm1.view(torch.int32))
    for u, v in zip(sums.tolist(), sums1.tolist()):
        assert abs(u - v) <= 1e-6 * abs(v)
    del bm1
    pick = np.unique(np.concatenate([np.arange(4), np.random.default_rng(94).choice(rows, 60, replace=False),
                                     np.arange(rows - 4, rows)]))
    idx = torch.from_numpy(pick).cuda()
    xs = host_view(x.index_select(0, idx))
    wc, ws = oracle.quantize(xs, "oas")
    assert_same_bits(c.index_select(0, idx), wc, "fused codes (sampled rows)")
    assert_same_bits(s.index_select(0, idx), ws, "fused scales (sampled rows)")
    assert_same_bits(y.index_select(0, idx), oracle.fakequant(xs, "oas"), "fused y (sampled rows)")
    wbm, _, _ = oracle.block_mse(xs, wc, ws, with_energy=True)
    assert np.allclose(bm.index_select(0, idx).cpu().numpy(), wbm, rtol=1e-6, atol=0)
    # the whole tensor: the oracle quantizes all 2^31 + 2^20 elements itself;
    # codes and scales equal everywhere, and the tensor sums agree
    say("fused big tensor: oracle over the whole tensor")
    del y
    xh = host_view(x)
    wc_all, ws_all = oracle.quantize(xh, "oas", threads=THREADS)
    assert_same_bits(s, ws_all, "fused scales (whole tensor)")
    assert_same_bits(c, wc_all, "fused codes (whole tensor)")
    _, wsse, wssq = oracle.block_mse(xh, wc_all, ws_all, threads=THREADS, with_energy=True)
    got = sums.tolist()
    assert same_sum(got[0], wsse) and same_sum(got[1], wssq), (got, wsse, wssq)


def test_fused_deterministic():
    """Repeated calls give the same bits, tensor sums included (fixed-order
    partial sums, no atomics)."""
    x = workloads.bf16_student_t_outlier_channels(63, shape=(2048, 4096)).cuda()
    first = mx.quantize_fused(x, "oas")
    for _ in range(3):
        again = mx.quantize_fused(x, "oas")
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
