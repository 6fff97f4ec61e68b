"""fp32 inputs at the rounding boundaries of the hardware converts, against the
oracle.

The fp32 paths round through gfx950's scaled converts, which are allowed only
where they match the oracle bit for bit. Every E2M1 rounding midpoint (0.25,
0.75, 1.25, 1.75, 2.5, 3.5, 5), the largest value 6 and the saturating range
(6, 8), times 2^(s-127) for every scale byte s, together with their two
nearest fp32 neighbours on each side, both signs, go through quantize,
dequantize, fake-quant and the one-pass call in all four scale modes (E2M1
grid and saturation: Axolotl MXFP4 PR page section 2; "Unveiling the Potential
of Quantization with MXFP4", technical summary section 2.A). The MBS-Static
and NVFP4 paths compute an fp32 value y before the same convert; their blocks
are built so that y equals x exactly (macro factor 1; block scale a power of
two), so the convert again sees the midpoints and their neighbours. MXFP8
gets every E4M3 midpoint and its saturating range the same way (vLLM
MXFP8/MXFP4 page, MXFP8 section).
"""
import os

import numpy as np
import pytest
import torch

import microscaling_fp4_block_mx_amd as mx
import oracle
from test_parity_gpu import THREADS, assert_same_bits, check_all_ops, host_view, say
from test_parity_mbs_gpu import check_mbs
from test_parity_mxfp8_gpu import check8
from test_parity_nvfp4_gpu import check_nv

pytestmark = pytest.mark.gpu

MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
TOP = (6.0, 6.5, 7.0, 7.5, 7.75)


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()
    oracle.build(force=not os.path.exists(os.path.join(os.path.dirname(oracle.__file__),
                                                       "libmxref.so")))
    yield
    torch.cuda.synchronize()


def neighbours(v: np.ndarray, k: int = 2) -> np.ndarray:
    """v (fp32) and its k nearest fp32 neighbours below and above."""
    out = [v]
    up, dn = v.copy(), v.copy()
    for _ in range(k):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(0))
        out += [up, dn]
    return np.concatenate(out).astype(np.float32)


def _fill(anchor_cols: dict, vals: np.ndarray, width: int, free_cols) -> np.ndarray:
    n = -(-vals.size // len(free_cols))
    pad = np.zeros(n * len(free_cols), np.float32)
    pad[:vals.size] = vals
    blk = np.zeros((n, width), np.float32)
    blk[:, free_cols] = pad.reshape(n, len(free_cols))
    for col, a in anchor_cols.items():
        blk[:, col] = a
    return blk


def e2m1_boundary_values(s: int) -> np.ndarray:
    base = (np.array(MIDS + TOP) * 2.0 ** (s - 127)).astype(np.float32)  # exact
    v = neighbours(base)
    return np.concatenate([v, -v])


def mxfp4_blocks() -> np.ndarray:
    """[n, 32]: anchor 4 * 2^(s-127) first (OCP byte s), then 31 values."""
    out = []
    for s in range(0, 253):
        a = np.float32(4.0 * 2.0 ** (s - 127))
        out.append(_fill({0: a}, e2m1_boundary_values(s), 32, list(range(1, 32))))
    return np.concatenate(out)


def test_mxfp4_fp32_rounding_boundaries_every_scale():
    # the inputs straddle the midpoints: the neighbours just below and just
    # above each midpoint round to different codes
    for s in (0, 1, 2, 127, 252):
        for m in MIDS:
            v = np.float32(m * 2.0 ** (s - 127))
            lo, hi = np.nextafter(v, np.float32(0)), np.nextafter(v, np.float32(np.inf))
            assert oracle.encode(float(lo), s) != oracle.encode(float(hi), s), (s, m)
    x = torch.from_numpy(mxfp4_blocks())
    check_all_ops(x, "fp32-boundaries")
    xd, xh = x.cuda(), host_view(x)
    for mode in ("ocp", "oas", "oas_bits", "oas_nf"):
        say(f"fp32-boundaries one-pass {mode}")
        c, s, y, bm, sums = mx.quantize_fused(xd, mode)
        wc, ws = oracle.quantize(xh, mode, threads=THREADS)
        assert_same_bits(s, ws, f"one-pass scales {mode}")
        assert_same_bits(c, wc, f"one-pass codes {mode}")
        assert_same_bits(y, oracle.dequantize(wc, ws, "f32", threads=THREADS), f"one-pass y {mode}")
        wbm, wsse, wssq = oracle.block_mse(xh, wc, ws, threads=THREADS, with_energy=True)
        np.testing.assert_allclose(bm.cpu().numpy(), wbm, rtol=1e-6, atol=0)
        got_sse, got_ssq = sums.tolist()
        assert abs(got_sse - wsse) <= 1e-6 * wsse and abs(got_ssq - wssq) <= 1e-6 * wssq


def mbs_macro_blocks() -> np.ndarray:
    """[n, 128]: sub-block 0 holds 12 * 2^(s-127) (a_M / 6 is a power of two,
    so the macro factor is 1 and y = x); sub-blocks 1..7 each hold the anchor
    4 * 2^(s-127) and 15 boundary values at byte s."""
    out = []
    free = [c for c in range(16, 128) if c % 16 != 0]
    for s in range(0, 251):  # 12 * 2^(s-127) is finite up to s = 250
        X = 2.0 ** (s - 127)
        anchors = {0: np.float32(12.0 * X)}
        anchors.update({16 * j: np.float32(4.0 * X) for j in range(1, 8)})
        out.append(_fill(anchors, e2m1_boundary_values(s), 128, free))
    return np.concatenate(out)


def test_mbs_static_fp32_rounding_boundaries():
    x = mbs_macro_blocks()
    _, _, mm = oracle.quantize_mbs(x)
    assert (mm == 0).all()  # every macro factor is 1: the convert sees x itself
    check_mbs(torch.from_numpy(x), "mbs-fp32-boundaries")


def nvfp4_tensors():
    """One [n, 16] tensor per range of 18 binades j in [J - 17, J]: blocks
    with the anchor 6 * 2^j (block scale 2^(j + t), exactly an E4M3 value, so
    x * S / s_b = x * 2^-j exactly) and 15 values m * 2^j near the E2M1
    midpoints, 6 and past it, both signs; plus blocks whose anchor 6.375 * 2^j
    makes the block scale round down (a tie in E4M3) and the top element
    saturate."""
    for J in range(125, -127, -18):
        rows = []
        for j in range(J - 17, J + 1):
            X = 2.0 ** j
            base = (np.array(MIDS + (5.5, 5.75, 6.0)) * X).astype(np.float32)
            v = neighbours(base)
            rows.append(_fill({0: np.float32(6.0 * X)}, np.concatenate([v, -v]), 16,
                              list(range(1, 16))))
            rows.append(_fill({0: np.float32(6.375 * X)},
                              (np.array(MIDS) * X).astype(np.float32), 16, list(range(1, 16))))
        yield J, np.concatenate(rows)


def test_nvfp4_fp32_rounding_boundaries():
    for J, x in nvfp4_tensors():
        _, _, t = oracle.quantize_nvfp4(x)
        assert t - 127 == 8 - J, (J, t)
        check_nv(torch.from_numpy(x), f"nvfp4-fp32-boundaries J={J}")


def _e4m3_magnitudes():
    v = []
    for c in range(1, 0x7F):
        e, m = c >> 3, c & 7
        v.append(np.ldexp(m / 8.0, -6) if e == 0 else np.ldexp(1.0 + m / 8.0, e - 7))
    return np.array(v)


def test_mxfp8_fp32_rounding_boundaries():
    g = _e4m3_magnitudes()
    mids = np.concatenate([[g[0] / 2], (g[:-1] + g[1:]) / 2, [448.0, 464.0, 480.0, 500.0, 511.0]])
    out = []
    for s in range(0, 247, 3):
        X = 2.0 ** (s - 127)
        v = neighbours((mids * X).astype(np.float32), 1)
        out.append(_fill({0: np.float32(256.0 * X)}, np.concatenate([v, -v]), 32,
                         list(range(1, 32))))
    check8(torch.from_numpy(np.concatenate(out)), "mxfp8-fp32-boundaries")
