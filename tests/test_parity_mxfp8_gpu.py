"""GPU parity of the MXFP8 (E4M3) kernels against the CPU oracle: codes,
scales, dequantized and fake-quantized values bit-exact. Inputs from
workloads/, expected values from oracle/ only."""
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


def check8(x: torch.Tensor, label: str):
    xh = host_view(x)
    xd = x.cuda()
    say(f"{label} mxfp8 {tuple(x.shape)} {x.dtype}")
    c, s = mx.quantize_mxfp8(xd)
    wc, ws = oracle.quantize_mxfp8(xh, threads=THREADS)
    assert_same_bits(s, ws, f"{label} mxfp8 scales")
    assert_same_bits(c, wc, f"{label} mxfp8 codes")
    for dt, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        assert_same_bits(mx.dequantize_mxfp8(c, s, dt),
                         oracle.dequantize_mxfp8(wc, ws, name, threads=THREADS),
                         f"{label} mxfp8 dequant {name}")
    assert_same_bits(mx.fakequant_mxfp8(xd), oracle.fakequant_mxfp8(xh, threads=THREADS),
                     f"{label} mxfp8 fakequant")


def exhaustive_blocks8():
    all_mag = np.arange(0, 0x7F80, dtype=np.uint32)
    out = []
    for s in range(0, 247):
        anchor = (s + 8) << 7
        limit = min((s + 9) << 7, 0x7F80)
        mags = all_mag[all_mag < limit]
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        n = -(-vals.size // 31)
        pad = np.zeros(n * 31, np.uint16)
        pad[:vals.size] = vals
        blk = np.empty((n, 32), np.uint16)
        blk[:, 0] = anchor
        blk[:, 1:] = pad.reshape(n, 31)
        out.append(blk)
    return np.concatenate(out, 0)


def test_mxfp8_exhaustive_bf16_every_scale():
    check8(workloads.from_bf16_bits(exhaustive_blocks8()), "exhaustive-bf16")


def test_mxfp8_exhaustive_fp32_widened():
    b = exhaustive_blocks8()
    check8(workloads.from_bf16_bits(b[::3].copy()).float(), "exhaustive-f32")


def test_mxfp8_special_and_wide():
    x = torch.from_numpy(workloads.special_blocks_f32())
    check8(x, "special-f32")
    check8(x.to(torch.bfloat16), "special-bf16")
    rng = np.random.default_rng(51)
    w = (rng.standard_normal((512, 64)) * np.ldexp(1.0, rng.integers(-149, 120, (512, 1))))
    check8(torch.from_numpy(w.astype(np.float32)), "wide-f32")


def test_mxfp8_dequantize_every_code_every_scale():
    codes = np.tile(np.arange(256, dtype=np.uint8), 256).reshape(256, 256)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 8, 1)
    cd, sd = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    for dt, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        assert_same_bits(mx.dequantize_mxfp8(cd, sd, dt), oracle.dequantize_mxfp8(codes, scales, name),
                         f"mxfp8 dequant all codes {name}")


@pytest.mark.parametrize("rows,k", [(1, 32), (3, 96), (257, 160), (1000, 4096), (4099, 64)])
def test_mxfp8_ragged(rows, k):
    rng = np.random.default_rng(rows * 7 + k)
    x = rng.laplace(0, 1, (rows, k)) * np.exp(rng.normal(0, 3, (rows, k // 32))).repeat(32, 1)
    x[rng.random((rows, k)) < 0.002] *= 500
    xt = torch.from_numpy(x.astype(np.float32))
    check8(xt, f"ragged-f32 {rows}x{k}")
    check8(xt.to(torch.bfloat16), f"ragged-bf16 {rows}x{k}")


def test_mxfp8_activations_full():
    check8(workloads.bf16_student_t_outlier_channels(2), "student-t 8192x4096")


def test_mxfp8_llama_linears_sampled_full():
    """Online MXFP8 quantization of the Llama-3.2-3B-shaped weights grouped by
    in_features; sampled rows against the oracle, the whole tensor against
    the fused fake-quant."""
    a, b = workloads.llama32_3b_grouped("cuda")
    for t, label, seed in ((a, "llama K=3072", 61), (b, "llama K=8192", 62)):
        say(f"{label} mxfp8 quantize")
        c, s = mx.quantize_mxfp8(t)
        rng = np.random.default_rng(seed)
        rows = np.unique(np.concatenate([np.arange(64), np.arange(t.shape[0] - 64, t.shape[0]),
                                         rng.choice(t.shape[0], 2048, replace=False)]))
        idx = torch.from_numpy(rows).cuda()
        wc, ws = oracle.quantize_mxfp8(host_view(t.index_select(0, idx)), threads=THREADS)
        assert_same_bits(c.index_select(0, idx), wc, f"{label} codes")
        assert_same_bits(s.index_select(0, idx), ws, f"{label} scales")
        y = mx.dequantize_mxfp8(c, s, torch.bfloat16)
        assert torch.equal(mx.fakequant_mxfp8(t).view(torch.int16), y.view(torch.int16))
        del c, s, y


def test_mxfp8_in_place_and_deterministic():
    x = workloads.bf16_laplace_sparse_outliers(8, shape=(2048, 8192)).cuda()
    c1, s1 = mx.quantize_mxfp8(x)
    c2, s2 = mx.quantize_mxfp8(x)
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    want = mx.fakequant_mxfp8(x)
    mx.fakequant_mxfp8(x, out=x)
    assert torch.equal(x.view(torch.int16), want.view(torch.int16))
