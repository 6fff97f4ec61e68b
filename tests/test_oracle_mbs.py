"""Pins of the oracle's MBS-Static variant: a hand-worked macro block, the
macro mantissa's closed form (including a tie), a re-derivation from numpy
fp32 arithmetic and an exact E2M1 search, and invariants."""
import numpy as np
import torch

import workloads
from conftest import golden_rows

G = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])


def test_golden_macro_block(oracle_lib):
    x = np.zeros((1, 128), np.float32)
    x[0, 0], x[0, 20], x[0, 40] = 7.5, 1.0, -0.3
    c, s, m = oracle_lib.quantize_mbs(x)
    y = oracle_lib.dequantize_mbs(c, s, m, "f32")
    head, dec = golden_rows("mbs_static_blocks.txt")[0].split("|")
    f = [int(v) for v in head.split()]
    assert m[0, 0] == f[0] and s[0].tolist() == f[1:]
    assert y[0, [0, 20, 40]].tolist() == [float(v) for v in dec.split()]


def test_macro_mantissa_closed_form(oracle_lib):
    for mm in (0, 1, 64, 127, 200, 255):
        for e in (-20, 0, 7):
            a = 6 * (1 + mm / 256) * 2.0 ** e
            assert oracle_lib.mbs_macro_mantissa(a) == mm
    # a_M / 6 = 1 + 64.5/256: tie between 64 and 65 -> 64 (even)
    assert oracle_lib.mbs_macro_mantissa(6 * (1 + 64.5 / 256)) == 64
    assert oracle_lib.mbs_macro_mantissa(6 * (1 + 65.5 / 256)) == 66
    # above 1 + 255.5/256 the rounding would carry; capped at 255
    assert oracle_lib.mbs_macro_mantissa(6 * (1 + 255.75 / 256)) == 255
    assert oracle_lib.mbs_macro_mantissa(0.0) == 0
    # a_M / 6 below half the smallest fp32 subnormal rounds to zero: factor 1
    for n in (1, 2, 3):
        assert oracle_lib.mbs_macro_mantissa(n * 2.0 ** -149) == 0
    # 4 * 2^-149 / 6 rounds to 2^-149 = 1.0 * 2^-149: mantissa 0 as well
    assert oracle_lib.mbs_macro_mantissa(4 * 2.0 ** -149) == 0
    # 7 * 2^-149 / 6 rounds to 2^-149 too; 9 * 2^-149 / 6 -> 2 * 2^-149 (tie, even)
    assert oracle_lib.mbs_macro_mantissa(7 * 2.0 ** -149) == 0
    assert oracle_lib.mbs_macro_mantissa(9 * 2.0 ** -149) == 0
    # 1.25 * 2^-140 * 6 is exact: subnormal a_M / 6 keeps its mantissa
    assert oracle_lib.mbs_macro_mantissa(6 * 1.25 * 2.0 ** -140) == 64
    x = np.zeros((1, 128), np.float32)
    x.view(np.uint32)[0, 0] = 3  # 3 * 2^-149
    x.view(np.uint32)[0, 1] = 0x80000001  # -2^-149
    c, s, m = oracle_lib.quantize_mbs(x)
    assert m[0, 0] == 0 and s[0, 0] == 0
    y = oracle_lib.dequantize_mbs(c, s, m, "f32")
    assert np.isfinite(y).all()
    # at byte 0 the grid step is 2^-128, so both round to zero (signs kept)
    assert (y[0, :2] == 0).all() and np.signbit(y[0, 1]) and not np.signbit(y[0, 0])


def _rederive(x: np.ndarray):
    xf = x.astype(np.float32).reshape(-1, 128)
    aM = np.abs(xf).max(1)
    r = (aM / np.float32(6)).astype(np.float32)
    mant, _ = np.frexp(r.astype(np.float64))
    t = (2 * mant - 1) * 256
    m = np.where(aM > 0, np.minimum(np.round(t), 255), 0).astype(np.int64)  # numpy rounds half even
    f = (np.float32(1) + m.astype(np.float32) / np.float32(256)).astype(np.float32)
    inv = (np.float32(1) / f).astype(np.float32)
    y = (xf * inv[:, None]).astype(np.float32).reshape(-1, 16)
    ay = np.abs(y).max(1).astype(np.float64)
    e = np.floor(np.log2(np.where(ay > 0, ay, 1)))
    s = np.where(ay > 0, np.clip(e - 2 + 127, 0, 254), 0).astype(np.int64)
    v = np.abs(y).astype(np.float64) / np.ldexp(1.0, s - 127)[:, None]
    d = np.abs(np.minimum(v, 6.0)[..., None] - G) * 4 + (np.arange(8) & 1) * 1e-9
    codes = np.argmin(d, -1) | (np.signbit(y) << 3)
    return codes.reshape(x.shape), s.reshape(x.shape[0], -1), m.reshape(x.shape[0], -1)


def test_rederivation_random(oracle_lib):
    rng = np.random.default_rng(81)
    for trial in range(4):
        x = (rng.standard_t(3, (32, 512)) * np.exp(rng.normal(0, 3, (32, 4))).repeat(128, 1)
             * 10.0 ** rng.integers(-15, 15)).astype(np.float32)
        c, s, m = oracle_lib.quantize_mbs(x)
        wc, ws, wm = _rederive(x)
        np.testing.assert_array_equal(m, wm)
        np.testing.assert_array_equal(s, ws)
        cc = np.empty(x.shape, np.int64)
        cc[:, 0::2] = c & 0xF
        cc[:, 1::2] = c >> 4
        np.testing.assert_array_equal(cc, wc)


def test_invariants(oracle_lib):
    rng = np.random.default_rng(82)
    x = (rng.standard_normal((16, 256)) * 5).astype(np.float32)
    c, s, m = oracle_lib.quantize_mbs(x)
    cn, sn, mn = oracle_lib.quantize_mbs(-x)
    np.testing.assert_array_equal(cn, c ^ 0x88)
    np.testing.assert_array_equal(sn, s)
    for j in (-9, 5):
        c2, s2, m2 = oracle_lib.quantize_mbs((x * np.float32(2.0 ** j)).astype(np.float32))
        np.testing.assert_array_equal(c2, c)
        np.testing.assert_array_equal(m2, m)
        np.testing.assert_array_equal(s2.astype(int), s.astype(int) + j)
    # decoding is exact: E2M1 * 2^(s-127) * (1 + m/256)
    y = oracle_lib.dequantize_mbs(c, s, m, "f32")
    cc = np.empty(x.shape, np.int64)
    cc[:, 0::2] = c & 0xF
    cc[:, 1::2] = c >> 4
    want = (np.where(cc & 8, -1, 1) * G[cc & 7] * np.ldexp(1.0, s.astype(np.int64) - 127).repeat(16, 1)
            * (1 + m.astype(np.float64) / 256).repeat(128, 1))
    np.testing.assert_array_equal(y, want.astype(np.float32))
    # the macro maximum decodes to within 2^-8 of itself (the factor's resolution)
    blocks = x.reshape(-1, 128)
    i = np.abs(blocks).argmax(1)
    got = y.reshape(-1, 128)[np.arange(blocks.shape[0]), i]
    ref = blocks[np.arange(blocks.shape[0]), i]
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8)


def test_special_values_and_bf16(oracle_lib):
    x = np.zeros((2, 128), np.float32)
    x[0, 7] = np.nan
    x[0, 70] = 3.0
    x[1] = np.linspace(-2, 2, 128)
    c, s, m = oracle_lib.quantize_mbs(x)
    assert s[0, 0] == 255 and s[0, 4] != 255
    y = oracle_lib.dequantize_mbs(c, s, m, "f32")
    assert (y[0, :16].view(np.uint32) == 0x7FC00000).all()
    # a NaN/Inf sub-block stores only the signs of its inputs (as an MXFP4
    # block with a NaN scale does), NaN signs included
    x2 = np.zeros((1, 128), np.float32)
    x2[0, 2], x2[0, 3], x2[0, 9] = -1.0, -np.inf, 5.0
    x2.view(np.uint32)[0, 5] = 0xFFC00000  # -NaN
    x2[0, 11] = -0.0
    c2, s2, m2 = oracle_lib.quantize_mbs(x2)
    assert s2[0, 0] == 255 and m2[0, 0] == 0
    nib = np.stack([c2[0, :8] & 15, c2[0, :8] >> 4], 1).reshape(-1)
    np.testing.assert_array_equal(nib, np.where(np.signbit(x2[0, :16]), 8, 0))
    xb = workloads.to_bf16_bits(torch.from_numpy(x[1:]).to(torch.bfloat16))
    cb, sb, mb = oracle_lib.quantize_mbs(xb)
    np.testing.assert_array_equal(oracle_lib.dequantize_mbs(cb, sb, mb, "bf16"),
                                  workloads.to_bf16_bits(torch.from_numpy(
                                      oracle_lib.dequantize_mbs(cb, sb, mb, "f32")).to(torch.bfloat16)))
