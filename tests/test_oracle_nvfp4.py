"""Pins of the oracle's NVFP4 comparator: hand-worked blocks, the tensor
factor's closed form, a re-derivation from independent library primitives
(numpy fp32 arithmetic, torch's float8_e4m3fn cast, exact E2M1 search) and
invariants."""
import numpy as np
import torch

import workloads
from conftest import golden_rows

G = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])


def test_golden_blocks(oracle_lib):
    x = np.zeros((1, 32), np.float32)
    x[0, :6] = [6, 3, 1.5, 0.5, -2, 4]
    x[0, 16] = 5
    codes, bs, ts = oracle_lib.quantize_nvfp4(x)
    assert ts == 135
    y = oracle_lib.dequantize_nvfp4(codes, bs, ts, "f32")
    c = np.empty(32, np.int64)
    c[0::2] = codes[0] & 0xF
    c[1::2] = codes[0] >> 4
    for row in golden_rows("nvfp4_blocks.txt"):
        head, dec = row.split("|")
        f = head.split()
        b = int(f[0])
        assert bs[0, b] == int(f[1], 16)
        assert [int(v, 16) for v in f[2:]] == c[16 * b:16 * b + 16].tolist()
        want = [float(v) for v in dec.split()]
        assert y[0, 16 * b:16 * b + len(want)].tolist() == want


def test_tensor_exponent_closed_form(oracle_lib):
    rng = np.random.default_rng(71)
    for a in np.ldexp(rng.uniform(1, 2, 500), rng.integers(-100, 100, 500)):
        t = oracle_lib.nvfp4_tensor_exp(a)
        assert a * 2.0 ** t <= 2688 < a * 2.0 ** (t + 1)
    assert oracle_lib.nvfp4_tensor_exp(0.0) == 0


def _rederive(x: np.ndarray):
    """Independent re-derivation on numpy fp32 arithmetic and torch's E4M3."""
    xf = x.astype(np.float32)
    fin = np.isfinite(xf)
    A = float(np.abs(np.where(fin, xf, 0)).max())
    t = 0
    if A > 0:
        t = int(np.floor(np.log2(2688.0 / A)))
        while A * 2.0 ** t > 2688:
            t -= 1
        while A * 2.0 ** (t + 1) <= 2688:
            t += 1
    S = np.float32(2.0 ** t)
    blk = xf.reshape(-1, 16)
    ab = np.abs(blk).max(1)
    tb = (ab / np.float32(6)).astype(np.float32) * S
    sb = torch.from_numpy(np.minimum(tb, 448).astype(np.float32)).to(torch.float8_e4m3fn)
    sbyte = sb.view(torch.uint8).numpy()
    sv = sb.float().numpy()
    r = np.where(sv > 0, (S / np.where(sv > 0, sv, 1)).astype(np.float32), np.float32(0))
    v = np.abs((blk * r[:, None]).astype(np.float32)).astype(np.float64)
    d = np.abs(np.minimum(v, 6.0)[..., None] - G) * 4 + (np.arange(8) & 1) * 1e-9
    idx = np.argmin(d, -1)
    codes = idx | (np.signbit(blk) << 3)
    return codes.reshape(x.shape), sbyte.reshape(x.shape[:-1] + (-1,)), t + 127


def test_rederivation_random(oracle_lib):
    rng = np.random.default_rng(72)
    for trial in range(6):
        scale = np.exp(rng.normal(0, 2, (64, 1))) * 10.0 ** rng.integers(-20, 20)
        x = (rng.standard_t(3, (64, 128)) * scale).astype(np.float32)
        codes, bs, ts = oracle_lib.quantize_nvfp4(x)
        wc, wb, wt = _rederive(x)
        assert ts == wt
        np.testing.assert_array_equal(bs, wb)
        c = np.empty(x.shape, np.int64)
        c[:, 0::2] = codes & 0xF
        c[:, 1::2] = codes >> 4
        np.testing.assert_array_equal(c, wc)


def test_invariants(oracle_lib):
    rng = np.random.default_rng(73)
    x = (rng.standard_normal((32, 64)) * 3).astype(np.float32)
    c, b, t = oracle_lib.quantize_nvfp4(x)
    cn, bn, tn = oracle_lib.quantize_nvfp4(-x)
    np.testing.assert_array_equal(cn, c ^ 0x88)
    np.testing.assert_array_equal(bn, b)
    for j in (-7, 3):
        c2, b2, t2 = oracle_lib.quantize_nvfp4((x * np.float32(2.0 ** j)).astype(np.float32))
        np.testing.assert_array_equal(c2, c)
        np.testing.assert_array_equal(b2, b)
        assert t2 == t - j
    y = oracle_lib.dequantize_nvfp4(c, b, t, "f32")
    # decoding is exact: (E2M1 * E4M3) / 2^t
    cc = np.empty(x.shape, np.int64)
    cc[:, 0::2] = c & 0xF
    cc[:, 1::2] = c >> 4
    sv = torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy().repeat(16, 1)
    want = np.where(cc & 8, -1, 1) * G[cc & 7] * sv / 2.0 ** (t - 127)
    np.testing.assert_array_equal(y, want.astype(np.float32))
    # the block maximum is reproduced to within half an E2M1 step of its block
    assert np.all(np.abs(y - x) <= np.abs(x).reshape(-1, 16).max(1).repeat(16).reshape(x.shape) * 0.25 + 1e-30)



def test_decode_every_block_scale_byte(oracle_lib):
    """Decoding reads the block scale as a full E4M3 byte, sign included
    (the quantizer never writes a negative one), against torch's own
    float8_e4m3fn reading of the byte: 0x7F and 0xFF are NaN."""
    rng = np.random.default_rng(77)
    bs = np.arange(256, dtype=np.uint8).reshape(16, 16)
    codes = rng.integers(0, 256, (16, 128), dtype=np.uint8)
    for t in (127, 135, 100):
        y = oracle_lib.dequantize_nvfp4(codes, bs, t, "f32")
        cc = np.empty((16, 256), np.int64)
        cc[:, 0::2] = codes & 0xF
        cc[:, 1::2] = codes >> 4
        sv = torch.from_numpy(bs).view(torch.float8_e4m3fn).float().numpy().astype(np.float64).repeat(16, 1)
        want = (np.where(cc & 8, -1, 1) * G[cc & 7] * sv / 2.0 ** (t - 127)).astype(np.float32)
        nan = np.isnan(sv)
        assert nan.sum() == 2 * 16 and np.isnan(y[nan]).all()
        np.testing.assert_array_equal(y[~nan], want[~nan])

def test_nonfinite_block_and_bf16(oracle_lib):
    x = np.zeros((2, 32), np.float32)
    x[0, 3] = np.nan
    x[0, 20] = 2.0
    x[1, :] = np.linspace(-1, 1, 32)
    c, b, t = oracle_lib.quantize_nvfp4(x)
    assert b[0, 0] == 0x7F and b[0, 1] != 0x7F
    y = oracle_lib.dequantize_nvfp4(c, b, t, "f32")
    assert (y[0, :16].view(np.uint32) == 0x7FC00000).all()
    xb = workloads.to_bf16_bits(torch.from_numpy(x[1:]).to(torch.bfloat16))
    cb, bb, tb = oracle_lib.quantize_nvfp4(xb)
    yb = oracle_lib.dequantize_nvfp4(cb, bb, tb, "bf16")
    yf = oracle_lib.dequantize_nvfp4(cb, bb, tb, "f32")
    np.testing.assert_array_equal(yb, workloads.to_bf16_bits(torch.from_numpy(yf).to(torch.bfloat16)))


def test_nvfp4_beats_mxfp4_on_weights(oracle_lib):
    """The pages' comparison: NVFP4's finer scale gives a lower error than
    MXFP4 OCP on N(0, 0.02) weights."""
    x = workloads.to_bf16_bits(workloads.bf16_normal(74, (256, 1024)))
    c, b, t = oracle_lib.quantize_nvfp4(x)
    ynv = workloads.from_bf16_bits(oracle_lib.dequantize_nvfp4(c, b, t, "bf16")).float().numpy()
    ymx = workloads.from_bf16_bits(oracle_lib.fakequant(x)).float().numpy()
    xf = workloads.from_bf16_bits(x).float().numpy()
    assert ((xf - ynv) ** 2).sum() < ((xf - ymx) ** 2).sum()


def test_block_scale_tie_and_tensor_boundary(oracle_lib):
    # hand-worked in tests/golden/nvfp4_blocks.txt (second tensor)
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 7.0
    x[0, 16] = 3.1875
    c, b, t = oracle_lib.quantize_nvfp4(x)
    assert t == 135 and b[0, 1] == 0x70
    assert (c[0, 8] & 0xF) == 7
    y = oracle_lib.dequantize_nvfp4(c, b, t, "f32")
    assert y[0, 16] == 3.0
    assert oracle_lib.nvfp4_tensor_exp(5.25) == 9
    assert oracle_lib.nvfp4_tensor_exp(5.25 * (1 + 2.0 ** -20)) == 8
    z = np.zeros((1, 16), np.float32)
    z[0, 2] = 5.25
    cz, bz, tz = oracle_lib.quantize_nvfp4(z)
    assert tz == 136
    # 5.25 * 2^9 = 2688 = 6 * 448 exactly: the block scale is E4M3's largest
    # finite value (torch reads byte 0x7E as 448) and the maximum is code 7
    assert bz[0, 0] == 0x7E
    assert torch.tensor([0x7E], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item() == 448.0
    assert (cz[0, 1] & 0xF) == 7
    assert oracle_lib.dequantize_nvfp4(cz, bz, tz, "f32")[0, 2] == 5.25


def test_signed_zero(oracle_lib):
    """E2M1's sign bit carries the sign of zero: -0.0 encodes to code 8 and
    decodes to -0.0 (fp32 bits 0x80000000), +0.0 to code 0, in a block
    with other values and in an all-zero block."""
    x = np.zeros((2, 16), np.float32)
    x[0, :4] = [-0.0, 0.0, 1.5, -0.0]
    x[1, :2] = [-0.0, 0.0]
    c, b, t = oracle_lib.quantize_nvfp4(x)
    assert (c[0, 0] & 0xF) == 8 and (c[0, 0] >> 4) == 0 and (c[0, 1] >> 4) == 8
    assert (c[1, 0] & 0xF) == 8 and (c[1, 0] >> 4) == 0
    y = oracle_lib.dequantize_nvfp4(c, b, t, "f32").view(np.uint32)
    assert y[0, 0] == 0x80000000 and y[0, 1] == 0 and y[0, 3] == 0x80000000
    assert y[1, 0] == 0x80000000 and y[1, 1] == 0
