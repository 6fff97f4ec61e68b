"""Pins of the oracle's MXFP8 (E4M3) path (vLLM MXFP8/MXFP4 page, MXFP8
section and MX format table) against torch's own float8_e4m3fn definition,
the format's closed forms and exhaustive enumeration."""
import math

import numpy as np
import torch

import workloads

E4M3_MAX = 448.0


def torch_e4m3_value(code: int) -> float:
    t = torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn)
    return float(t.float().item())


def e4m3_closed_form(code: int) -> float:
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def test_decode_table_matches_torch_and_closed_form(oracle_lib):
    for c in range(256):
        want = torch_e4m3_value(c)
        assert (math.isnan(want) and math.isnan(e4m3_closed_form(c))) or \
            want == e4m3_closed_form(c), c
        got = oracle_lib.decode_e4m3(c, 127)
        assert (math.isnan(got) and math.isnan(want)) or got == want, c
    assert e4m3_closed_form(0x7E) == E4M3_MAX


def test_decode_all_codes_all_scales(oracle_lib):
    for s in range(255):
        for c in range(0, 256, 3):
            want = e4m3_closed_form(c)
            got = oracle_lib.decode_e4m3(c, s)
            if math.isnan(want):
                assert math.isnan(got)
            else:
                assert got == math.ldexp(want, s - 127), (c, s)
    assert math.isnan(oracle_lib.decode_e4m3(0x10, 255))


def test_scale_rule_every_bf16_lone_element(oracle_lib):
    h = np.arange(0x0001, 0x7F80, dtype=np.uint16)
    x = np.zeros((h.size, 32), np.uint16)
    x[:, 3] = h
    _, scales = oracle_lib.quantize_mxfp8(x)
    e = (h.astype(np.int32) >> 7) & 0xFF
    want = np.maximum(e - 8, 0)  # floor(log2) - 8 + 127 = exponent field - 8
    np.testing.assert_array_equal(scales[:, 0].astype(np.int32), want)


def _torch_reference_codes(v: np.ndarray) -> np.ndarray:
    """E4M3 codes of float32 values v (already divided by the block scale):
    torch's round-to-nearest-even cast after clamping to +-448."""
    t = torch.from_numpy(np.clip(v, -E4M3_MAX, E4M3_MAX).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_exhaustive_bf16_every_scale_vs_torch(oracle_lib):
    """Every bf16 magnitude below 512 * 2^(s-127), both signs, behind an
    anchor 256 * 2^(s-127), for every scale byte s the rule can produce."""
    all_mag = np.arange(0, 0x7F80, dtype=np.uint32)
    for s in list(range(0, 247, 1)):
        anchor = (s + 8) << 7          # 256 * 2^(s-127) has exponent field s+8
        limit = (s + 9) << 7
        if limit > 0x7F80:
            break
        mags = all_mag[all_mag < limit]
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        n = -(-vals.size // 31)
        pad = np.zeros(n * 31, np.uint16)
        pad[:vals.size] = vals
        blk = np.empty((n, 32), np.uint16)
        blk[:, 0] = anchor
        blk[:, 1:] = pad.reshape(n, 31)
        codes, scales = oracle_lib.quantize_mxfp8(blk)
        assert (scales == s).all(), s
        xf = workloads.from_bf16_bits(blk).float().numpy().astype(np.float64)
        v = (xf / 2.0 ** (s - 127)).astype(np.float32)  # exact power-of-two division
        want = _torch_reference_codes(v)
        # torch keeps the sign of zero the same way (sign bit set for -0)
        np.testing.assert_array_equal(codes, want, err_msg=f"scale byte {s}")


def test_fp32_random_vs_torch(oracle_lib):
    rng = np.random.default_rng(41)
    x = (rng.standard_t(3, (2048, 64)) * np.ldexp(1.0, rng.integers(-120, 110, (2048, 1)))).astype(np.float32)
    codes, scales = oracle_lib.quantize_mxfp8(x)
    X = np.ldexp(1.0, scales.astype(np.int64) - 127).repeat(32, 1)
    want = _torch_reference_codes((x.astype(np.float64) / X).astype(np.float32))
    np.testing.assert_array_equal(codes, want)


def test_saturation_and_ties(oracle_lib):
    # at scale 1: 448 exact, 456 (between 448 and the absent 480) -> 448,
    # 500 -> 448; 2^-10 is a tie between 0 and 2^-9 -> 0 (even)
    for v, want in ((448.0, 0x7E), (456.0, 0x7E), (500.0, 0x7E), (2.0 ** -10, 0x00),
                    (3 * 2.0 ** -10, 0x02), (1.0, 0x38), (1.0625, 0x38), (1.1875, 0x3A),
                    (-2.0 ** -12, 0x80)):
        assert oracle_lib.encode_e4m3(v, 127) == want, v


def test_roundtrip_all_representable(oracle_lib):
    rows = []
    for s in range(0, 240, 7):
        X = math.ldexp(1.0, s - 127)
        row = [256 * X] + [e4m3_closed_form(c) * X for c in range(1, 32)]
        rows.append(row)
        row = [256 * X] + [e4m3_closed_form(c) * X for c in range(96, 127)]
        rows.append(row)
    x = np.array(rows, np.float32)
    codes, scales = oracle_lib.quantize_mxfp8(x)
    np.testing.assert_array_equal(oracle_lib.dequantize_mxfp8(codes, scales, "f32"), x)
    np.testing.assert_array_equal(oracle_lib.fakequant_mxfp8(x), x)


def test_special_blocks(oracle_lib):
    x = workloads.special_blocks_f32()
    codes, scales = oracle_lib.quantize_mxfp8(x)
    y = oracle_lib.dequantize_mxfp8(codes, scales, "f32")
    assert scales[0, 0] == 0 and (codes[0] == 0).all()
    assert (codes[1] == 0x80).all() and np.signbit(y[1]).all()
    for r in (2, 3, 4):
        assert scales[r, 0] == 255
        assert (codes[r] == np.where(np.signbit(x[r]), 0x80, 0)).all()
        assert (y[r].view(np.uint32) == 0x7FC00000).all()
    np.testing.assert_array_equal(oracle_lib.fakequant_mxfp8(x).view(np.uint32), y.view(np.uint32))


def test_bf16_output_rounding_of_tiny_values(oracle_lib):
    """At scale bytes 0..3 some E4M3 values fall below bf16's subnormal step
    (2^-133); the bf16 output is torch's round-to-nearest-even cast of the
    exact fp32 value."""
    codes = np.tile(np.arange(256, dtype=np.uint8), 4).reshape(4, 256)  # 8 blocks per row
    for s in range(4):
        scales = np.full((4, 8), s, np.uint8)
        f = oracle_lib.dequantize_mxfp8(codes, scales, "f32")
        b = oracle_lib.dequantize_mxfp8(codes, scales, "bf16")
        want = workloads.to_bf16_bits(torch.from_numpy(f).to(torch.bfloat16))
        nan = np.isnan(f)
        np.testing.assert_array_equal(b[~nan], want[~nan])
        assert (b[nan] == 0x7FC0).all()
