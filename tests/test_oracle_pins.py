"""Pins of the CPU oracle against what the format and mathematics fix.

Nothing here re-types the oracle's formulas: every expectation comes from an
independent derivation (bit-field closed forms of E2M1/E8M0, an exact integer
or rational nearest-grid brute force, torch's own E8M0 byte interpretation,
hand-worked blocks under tests/golden/ with their derivations, invariants).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from conftest import golden_rows

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
        Fraction(3), Fraction(4), Fraction(6)]


def e2m1_closed_form(code):
    """S1E2M1 bit interpretation: bit 3 sign, bits 2..1 exponent (bias 1),
    bit 0 mantissa; exponent 0 is subnormal (m * 0.5)."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def exact_nearest_index(q: Fraction) -> int:
    """Brute force: index of the E2M1 magnitude nearest to q >= 0, exact
    rational distances, ties to the even index."""
    best = None
    for i, g in enumerate(GRID):
        key = (abs(q - g), i & 1)
        if best is None or key < best[0]:
            best = (key, i)
    return best[1]


def bf16_exact(h: int) -> Fraction:
    e, m = (h >> 7) & 0xFF, h & 0x7F
    mag = Fraction(m, 1) * Fraction(2) ** -133 if e == 0 else \
        Fraction(128 + m) * Fraction(2) ** (e - 134)
    return -mag if h & 0x8000 else mag


def f32_exact(x: float) -> Fraction:
    return Fraction(float(np.float32(x)))


# ---- element format --------------------------------------------------------

def test_e2m1_table_closed_form(oracle_lib):
    assert [e2m1_closed_form(c) for c in range(8)] == GRID
    for c in range(16):
        assert Fraction(oracle_lib.decode(c, 127)) == e2m1_closed_form(c), c


def test_decode_all_codes_all_scales(oracle_lib):
    # 16 codes x 255 finite scale bytes = 4080 values vs exact ldexp
    for s in range(255):
        for c in range(16):
            want = e2m1_closed_form(c) * Fraction(2) ** (s - 127)
            got = oracle_lib.decode(c, s)
            assert Fraction(got) == want, (c, s)
    assert math.isnan(oracle_lib.decode(3, 255))


def test_e8m0_bias_matches_torch_byte_view(oracle_lib):
    # torch.float8_e8m0fnu is an independent definition of the E8M0 byte.
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for s in range(255):
        assert oracle_lib.decode(2, s) == ref[s], s  # code 2 is +1.0
    assert math.isnan(ref[255]) and math.isnan(oracle_lib.decode(2, 255))


# ---- scale rule ------------------------------------------------------------

def test_ocp_scale_every_bf16_lone_element(oracle_lib):
    # Every finite bf16 pattern as the only nonzero element of a block.
    h = np.arange(0x0000, 0x7F80, dtype=np.uint16)
    h = np.concatenate([h, h | 0x8000])
    x = np.zeros((h.size, 32), np.uint16)
    x[:, 7] = h
    _, scales = oracle_lib.quantize(x)
    expfield = (h.astype(np.int32) >> 7) & 0xFF
    want = np.maximum(expfield - 2, 0)
    want[(h & 0x7FFF) == 0] = 0
    np.testing.assert_array_equal(scales[:, 0].astype(np.int32), want)


def test_ocp_scale_normalizes_amax_into_4_8(oracle_lib):
    rng = np.random.default_rng(11)
    xs = np.ldexp(rng.uniform(1, 2, 3000), rng.integers(-120, 120, 3000)).astype(np.float32)
    for x in xs:
        s = oracle_lib.ocp_scale(float(x))
        assert 0 < s <= 252
        v = f32_exact(x) / Fraction(2) ** (s - 127)
        assert 4 <= v < 8, (x, s)


def test_scale_range_ends(oracle_lib):
    big = float(np.finfo(np.float32).max)
    assert oracle_lib.ocp_scale(big) == 252
    assert oracle_lib.ocp_scale(float(workloads.from_bf16_bits(np.array([0x7F7F], np.uint16)).float())) == 252
    for e in (-126, -130, -140, -149):
        assert oracle_lib.ocp_scale(math.ldexp(1.0, e)) == 0
    assert oracle_lib.ocp_scale(math.ldexp(1.0, -125)) == 0
    assert oracle_lib.ocp_scale(math.ldexp(1.0, -124)) == 1
    assert oracle_lib.ocp_scale(0.0) == 0
    # past fp32's range (a double argument) the byte stops at E8M0's largest
    # finite scale 2^127; byte 255 is E8M0's NaN, never a clamp
    for e in (128, 129, 130, 131, 200, 1000):
        assert oracle_lib.ocp_scale(math.ldexp(1.0, e)) == min(e - 2 + 127, 254), e


# ---- rounding --------------------------------------------------------------

def test_tie_table_golden(oracle_lib):
    for row in golden_rows("e2m1_ties.txt"):
        v, code, val = row.split()
        assert oracle_lib.encode(float(v), 127) == int(code), row
        got = oracle_lib.decode(int(code), 127)
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_exhaustive_bf16_all_scales_exact_integer_bruteforce(oracle_lib):
    """Every bf16 magnitude below 8*2^(s-127), both signs, for every scale
    byte s in [0, 252], against an exact integer nearest-grid computation."""
    grid_q = np.array([0, 1, 2, 3, 4, 6, 8, 12], np.int64) << 15  # GRID * 2^16
    blocks = workloads.exhaustive_bf16_blocks(range(0, 253))
    codes, scales = oracle_lib.quantize(blocks)
    # which s each block was built for: its anchor's exponent field minus 2
    s_blk = ((blocks[:, 0].astype(np.int64) >> 7) & 0xFF) - 2
    np.testing.assert_array_equal(scales[:, 0].astype(np.int64), s_blk)
    c = np.empty((blocks.shape[0], 32), np.int64)
    c[:, 0::2] = codes & 0xF
    c[:, 1::2] = codes >> 4
    h = blocks.astype(np.int64)
    s = np.repeat(s_blk[:, None], 32, 1)
    e, m = (h >> 7) & 0xFF, h & 0x7F
    mant = np.where(e == 0, m, 128 + m)
    p = np.where(e == 0, -133, e - 134) + 127 - s  # |x|/X = mant * 2^p
    sh = p + 16
    V = np.where(sh >= 0, mant << np.clip(sh, 0, 62), 0)  # exact (|x|/X) * 2^16
    small = sh < 0  # |x|/X < 2^-8: nearest is 0
    dist = np.abs(V[..., None] - grid_q) * 2 + (np.arange(8) & 1)
    idx = np.argmin(dist, axis=-1)
    idx[small] = 0
    want = idx | ((h >> 15) << 3)
    np.testing.assert_array_equal(c, want)


def test_fp32_random_fraction_bruteforce(oracle_lib):
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((64, 32)) * np.ldexp(1.0, rng.integers(-140, 120, (64, 1)))).astype(np.float32)
    x[3, :8] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 8.0]
    codes, scales = oracle_lib.quantize(x)
    for r in range(x.shape[0]):
        s = int(scales[r, 0])
        X = Fraction(2) ** (s - 127)
        amax = max(abs(f32_exact(v)) for v in x[r])
        # scale: the largest byte b with 4*2^(b-127) <= amax, floored at 0
        b = 0
        while b < 254 and 4 * Fraction(2) ** (b + 1 - 127) <= amax:
            b += 1
        assert s == b, r
        for i in range(32):
            code = (codes[r, i // 2] >> (4 * (i % 2))) & 0xF
            q = abs(f32_exact(x[r, i])) / X
            want = exact_nearest_index(q) | (8 if np.signbit(x[r, i]) else 0)
            assert code == want, (r, i, x[r, i])


def test_packing_golden(oracle_lib):
    rows = dict(line.split(":", 1) for line in golden_rows("packing_block.txt"))
    x = np.array([float(v) for v in rows["input"].split()], np.float32)[None]
    codes, scales = oracle_lib.quantize(x)
    assert int(scales[0, 0]) == int(rows["scale"])
    assert [int(b, 16) for b in rows["codes"].split()] == codes[0].tolist()
    # unpack(pack(c)) == c via the dequantizer
    y = oracle_lib.dequantize(codes, scales, "f32")
    np.testing.assert_array_equal(y, x)


def test_exact_roundtrip_all_representable(oracle_lib):
    """+-G * 2^(s-127) for all 15 nonzero codes and s in [0, 252] come back
    with the same code and scale, and dequantize exactly."""
    rows = []
    for s in range(253):
        X = math.ldexp(1.0, s - 127)
        row = [4 * X] + [float(e2m1_closed_form(c)) * X if c != 8 else -0.0
                         for c in range(1, 16)] + [0.0] * 16
        rows.append(row)
    x = np.array(rows, np.float32)
    codes, scales = oracle_lib.quantize(x)
    assert scales[:, 0].tolist() == list(range(253))
    for c in range(1, 16):
        i = c
        got = (codes[:, i // 2] >> (4 * (i % 2))) & 0xF
        assert (got == c).all(), c
    np.testing.assert_array_equal(oracle_lib.dequantize(codes, scales, "f32"), x)
    xb = workloads.to_bf16_bits(torch.from_numpy(x).to(torch.bfloat16))
    cb, sb = oracle_lib.quantize(xb)
    np.testing.assert_array_equal(cb, codes)
    np.testing.assert_array_equal(oracle_lib.dequantize(cb, sb, "bf16"), xb)


# ---- special cases ---------------------------------------------------------

def test_special_blocks(oracle_lib):
    x = workloads.special_blocks_f32()
    codes, scales = oracle_lib.quantize(x)
    y = oracle_lib.dequantize(codes, scales, "f32")
    # all zero / all -0
    assert scales[0, 0] == 0 and (codes[0] == 0).all() and (y[0] == 0).all()
    assert scales[1, 0] == 0 and (codes[1] == 0x88).all()
    assert np.signbit(y[1]).all()
    # NaN / +-Inf blocks: byte 255, sign-only codes, canonical NaN out
    for r in (2, 3, 4):
        assert scales[r, 0] == 255
        sign = np.signbit(x[r]).astype(np.uint8) * 8
        assert (codes[r] == (sign[0::2] | (sign[1::2] << 4))).all()
        assert (y[r].view(np.uint32) == 0x7FC00000).all()
    # lone 2^-128 (fp32 subnormal): byte 0, scale 2^-127, value 0.5 -> code 1
    assert scales[5, 0] == 0 and codes[5, 0] == 0x01
    # 2^-149 and -3*2^-149: byte 0, both far below 0.25*2^-127 -> 0 / -0
    assert scales[6, 0] == 0 and codes[6, 0] == 0x80
    # largest fp32: byte 252; max/2^125 ~ 7.99 saturates to 6 (code 7)
    assert scales[7, 0] == 252 and (codes[7, 0] & 0xF) == 7
    # 1.5*2^-126 and 2^-127 at byte 0 (scale 2^-127): 3.0 -> code 5, 1.0 -> code 2
    assert scales[12, 0] == 0 and codes[12, 0] == 0x25


def test_all_amax_below_clamp(oracle_lib):
    x = np.zeros((1, 32), np.float32)
    x[0, :] = np.ldexp(np.float32(1.75), -126)
    codes, scales = oracle_lib.quantize(x)
    # 1.75*2^-126 / 2^-127 = 3.5 -> tie between 3 and 4 -> 4 (code 6)
    assert scales[0, 0] == 0 and (codes[0] == 0x66).all()


# ---- invariants ------------------------------------------------------------

def _rand(seed, shape=(256, 128)):
    rng = np.random.default_rng(seed)
    return (rng.standard_t(3, shape) * np.exp(rng.normal(0, 2, (shape[0], 1)))).astype(np.float32)


def test_sign_symmetry(oracle_lib):
    x = _rand(1)
    c, s = oracle_lib.quantize(x)
    cn, sn = oracle_lib.quantize(-x)
    np.testing.assert_array_equal(s, sn)
    np.testing.assert_array_equal(cn, c ^ 0x88)


def test_scale_equivariance(oracle_lib):
    x = _rand(2)
    c, s = oracle_lib.quantize(x)
    for k in (-20, -3, 1, 7):
        c2, s2 = oracle_lib.quantize((x * np.float32(2.0 ** k)).astype(np.float32))
        np.testing.assert_array_equal(c2, c)
        np.testing.assert_array_equal(s2.astype(int), s.astype(int) + k)


def test_permutation_within_block(oracle_lib):
    x = _rand(3, (64, 32))
    perm = np.random.default_rng(4).permutation(32)
    c, s = oracle_lib.quantize(x)
    cp, sp = oracle_lib.quantize(np.ascontiguousarray(x[:, perm]))
    np.testing.assert_array_equal(s, sp)
    y = oracle_lib.dequantize(c, s, "f32")
    yp = oracle_lib.dequantize(cp, sp, "f32")
    np.testing.assert_array_equal(y[:, perm], yp)


def test_monotone_within_block(oracle_lib):
    x = np.sort(_rand(5, (64, 32)), axis=1)
    y = oracle_lib.fakequant(x)
    assert (np.diff(y, axis=1) >= 0).all()


def test_fakequant_idempotent_and_equals_roundtrip(oracle_lib):
    for mode in ("ocp", "oas"):
        x = _rand(6)
        y = oracle_lib.fakequant(x, mode)
        c, s = oracle_lib.quantize(x, mode)
        np.testing.assert_array_equal(y, oracle_lib.dequantize(c, s, "f32"))
        np.testing.assert_array_equal(oracle_lib.fakequant(y, mode), y)
        xb = workloads.to_bf16_bits(torch.from_numpy(x).to(torch.bfloat16))
        yb = oracle_lib.fakequant(xb, mode)
        np.testing.assert_array_equal(oracle_lib.fakequant(yb, mode), yb)


def test_error_bound(oracle_lib):
    x = _rand(7)
    c, s = oracle_lib.quantize(x)
    y = oracle_lib.dequantize(c, s, "f32").astype(np.float64)
    X = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    ax = np.abs(x.astype(np.float64))
    # half the local grid gap: 0.25X below 2X, 0.5X below 4X, X above
    half_gap = np.where(ax < 2 * X, 0.25 * X, np.where(ax < 4 * X, 0.5 * X, X))
    bound = np.maximum(half_gap, ax - 6 * X)
    assert (np.abs(ax - np.abs(y)) <= bound).all()


# ---- overflow-aware mode ---------------------------------------------------

def test_oas_worked_blocks_golden(oracle_lib):
    for row in golden_rows("oas_worked_blocks.txt"):
        name, n, sse0, sse1, byte = row.split()
        x = np.zeros(32, np.float32)
        x[0] = 4.0
        x[1:1 + int(n)] = 0.75
        # both errors in units of the larger candidate's scale (here 1)
        assert oracle_lib.oas_sse32(x.astype(np.float64), 127, 127) == float(sse0)
        assert oracle_lib.oas_sse32(x.astype(np.float64), 126, 127) == float(sse1)
        _, s = oracle_lib.quantize(x[None], "oas")
        assert int(s[0, 0]) == int(byte), name
        _, s = oracle_lib.quantize(x[None], "ocp")
        assert int(s[0, 0]) == 127


def test_overflow_aware_choice_at_the_ends_of_the_byte_range(oracle_lib):
    """The worked blocks of tests/golden/oas_worked_blocks.txt (A: 4 and
    sixteen 0.75, a tie, keeps the OCP byte; B: seventeen 0.75 takes one
    byte less) scaled by 2^(s-127) down to the smallest byte that has a
    smaller candidate (s = 1, where the 0.75 * 2^-126 elements are fp32
    subnormals, still exact) and up to the largest (252): every term of
    both errors is the same in units of the larger candidate, so the choice
    is the worked one. Likewise block C = {3.25, five 0.75} for the
    no-overflow pair: at its no-overflow byte 3.25 rounds to 3 (error 0.25)
    and each 0.75 ties to 1 (0.25), SSE 0.375; one byte lower 6.5
    saturates to 6 (0.25 in the same units) and 1.5 is exact, SSE 0.0625:
    the smaller byte wins, also at no-overflow byte 1."""
    for s in (1, 2, 127, 251, 252):
        for n, want in ((16, s), (17, s - 1)):
            x = np.zeros((1, 32), np.float32)
            x[0, 0] = 4.0
            x[0, 1:1 + n] = 0.75
            x = (x * np.float32(2.0 ** (s - 127))).astype(np.float32)
            assert Fraction(float(x[0, 0])) == 4 * Fraction(2) ** (s - 127)
            assert Fraction(float(x[0, 1])) == Fraction(3, 4) * Fraction(2) ** (s - 127)
            _, so = oracle_lib.quantize(x, "ocp")
            _, sa = oracle_lib.quantize(x, "oas")
            assert int(so[0, 0]) == s and int(sa[0, 0]) == want, (s, n)
    for s in (1, 2, 127, 252):
        x = np.zeros((1, 32), np.float32)
        x[0, 3] = 3.25
        x[0, 10:15] = 0.75
        x = (x * np.float32(2.0 ** (s - 127))).astype(np.float32)
        assert Fraction(float(x[0, 3])) == Fraction(13, 4) * Fraction(2) ** (s - 127)
        assert Fraction(float(x[0, 10])) == Fraction(3, 4) * Fraction(2) ** (s - 127)
        _, sn = oracle_lib.quantize(x, "oas_nf")
        _, sb = oracle_lib.quantize(x, "oas_bits")
        assert int(sn[0, 0]) == s - 1 and int(sb[0, 0]) == s - 1, s


def test_oas_never_worse_than_ocp(oracle_lib):
    x = workloads.to_bf16_bits(workloads.bf16_laplace_sparse_outliers(seed=9, shape=(64, 4096)))
    co, so = oracle_lib.quantize(x, "ocp")
    ca, sa = oracle_lib.quantize(x, "oas")
    bo, _ = oracle_lib.block_mse(x, co, so)
    ba, _ = oracle_lib.block_mse(x, ca, sa)
    assert (ba <= bo * (1 + 1e-6)).all()
    assert ((sa == so) | (sa.astype(int) == so.astype(int) - 1)).all()


def test_oas_decision_vs_exact_rational(oracle_lib):
    """Tiny dyadic blocks: the pinned fp32 decision equals the exact decision
    wherever the exact SSE gap exceeds fp32 rounding."""
    rng = np.random.default_rng(13)
    picked_low = kept = 0
    # values that sit on ties at scale 1 but on the grid at scale 1/2, mixed
    # with generic eighths, and a top element near 4 so both choices occur
    # (0.25 and 0.75 cost 0.0625 each at scale 1 and nothing at scale 1/2,
    # while a top element of 4 costs 1.0 at scale 1/2)
    tie_prone = np.array([0.25, 0.75, 0.75, 0.5, 1.0, 1.25, 0.0])
    for _ in range(400):
        n_tie = rng.integers(8, 33)
        x = (rng.integers(-8, 9, 32) / 8.0).astype(np.float32)
        x[:n_tie] = rng.choice(tie_prone, n_tie) * rng.choice([-1.0, 1.0], n_tie)
        x[rng.integers(32)] = rng.choice([4.0, 4.0, 4.125, -4.0, 5.0, 7.5])
        x *= np.float32(2.0 ** rng.integers(-20, 20))
        _, s = oracle_lib.quantize(x[None], "oas")
        s0 = oracle_lib.ocp_scale(float(np.abs(x).max()))

        def sse(b):
            X = Fraction(2) ** (b - 127)
            tot = Fraction(0)
            for v in x:
                q = GRID[exact_nearest_index(abs(f32_exact(v)) / X)] * X
                tot += (abs(f32_exact(v)) - q) ** 2
            return tot
        e0, e1 = sse(s0), sse(s0 - 1)
        if abs(e0 - e1) > Fraction(1, 2 ** 16) * max(e0, e1):
            want = s0 - 1 if e1 < e0 else s0
            assert int(s[0, 0]) == want
            picked_low += want == s0 - 1
            kept += want == s0
    assert picked_low >= 5 and kept >= 5


# ---- error measure ---------------------------------------------------------

def test_mse_zero_on_representable(oracle_lib):
    x = np.array([[0.5, 1, 1.5, 2, 3, 4, 6, -0.5] * 4], np.float32)
    c, s = oracle_lib.quantize(x)
    bm, sse = oracle_lib.block_mse(x, c, s)
    assert bm[0, 0] == 0.0 and sse == 0.0


def test_mse_closed_form(oracle_lib):
    # a lone 5*X -> 4*X (tie to even) gives SSE = X^2, block MSE = X^2/32
    for s in (3, 100, 127, 200):
        X = math.ldexp(1.0, s - 127)
        x = np.zeros((1, 32), np.float32)
        x[0, 9] = 5 * X
        c, sc = oracle_lib.quantize(x)
        assert sc[0, 0] == s
        bm, sse = oracle_lib.block_mse(x, c, sc)
        # the fp32 block MSE of an SSE beyond fp32's range (s = 200: 2^141)
        # is +Inf, IEEE conversion of the fp64 quotient
        want = np.float32(X * X / 32) if X * X / 32 < 2.0 ** 128 else np.float32(np.inf)
        assert sse == X * X and bm[0, 0] == want



def test_mse_reconstruction_overflows_like_fp32(oracle_lib):
    """The error is taken against the value an fp32 dequantize returns: at
    byte 254 a code of magnitude 2 or more decodes past fp32's largest finite
    value (2^128 > (2 - 2^-23) * 2^127), so the reconstruction is +Inf and so
    is the tensor SSE; one byte lower it is 2^127, finite."""
    for dt in ("f32", "bf16"):
        x = np.ones((1, 32), np.float32)
        if dt == "bf16":
            x = workloads.to_bf16_bits(torch.from_numpy(x).to(torch.bfloat16))
        codes = np.full((1, 16), 0x44, np.uint8)          # every element: +2.0
        for byte, want in ((253, 32 * 2.0 ** 254), (254, math.inf)):
            bm, sse = oracle_lib.block_mse(x, codes, np.full((1, 1), byte, np.uint8))
            # d = 1 - 2^127 rounds to -2^127 in fp64: SSE = 32 * 2^254 exactly
            assert sse == want, (dt, byte, sse)
            assert bm[0, 0] == np.float32(np.inf)           # 2^254 is past fp32 either way

def test_mse_matches_mean_of_squares(oracle_lib):
    x = _rand(8)
    c, s = oracle_lib.quantize(x)
    y = oracle_lib.dequantize(c, s, "f32").astype(np.float64)
    bm, sse = oracle_lib.block_mse(x, c, s)
    d2 = (x.astype(np.float64) - y) ** 2
    np.testing.assert_allclose(bm, d2.reshape(x.shape[0], -1, 32).mean(-1), rtol=1e-7)
    assert abs(sse - d2.sum()) <= 1e-12 * d2.sum()
    # the energy beside it (QSNR's numerator): every element's square, once
    _, sse2, ssq = oracle_lib.block_mse(x, c, s, with_energy=True)
    x2 = x.astype(np.float64) ** 2
    assert sse2 == sse and abs(ssq - x2.sum()) <= 1e-12 * x2.sum()
    # and per row: a tensor of one nonzero row carries exactly that row's energy
    for r in (0, x.shape[0] - 1):
        xr = np.zeros_like(x)
        xr[r] = x[r]
        cr, sr = oracle_lib.quantize(xr)
        _, _, ssq_r = oracle_lib.block_mse(xr, cr, sr, with_energy=True)
        assert abs(ssq_r - x2[r].sum()) <= 1e-12 * x2[r].sum()


def test_footprint_closed_form():
    rows = golden_rows("footprint.txt")
    params, gib, pct = rows[0].split()
    n = float(params)
    codes_bytes = n / 2
    assert round(codes_bytes / 1024 ** 3) == int(gib)
    assert round(100 / 32) == int(pct)  # 8-bit elements: 1 byte per 32 bytes
    assert (n / 2 + n / 32) * 8 / n == 4.25  # bits per element with scales


def test_threads_do_not_change_results(oracle_lib):
    x = _rand(10, (97, 256))
    a = oracle_lib.quantize(x, "oas", threads=1)
    b = oracle_lib.quantize(x, "oas", threads=5)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    ba = oracle_lib.block_mse(x, *a, threads=1)
    bb = oracle_lib.block_mse(x, *a, threads=7)
    np.testing.assert_array_equal(ba[0], bb[0])


def test_bad_shape_rejected(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.quantize(np.zeros((2, 48), np.float32))
