"""Pins of the oracle's page-faithful overflow-aware modes and of the QSNR
sums ("Unveiling the Potential of Quantization with MXFP4", technical summary
sections 2.A and 3-4), against hand-worked blocks and exact rationals."""
import math
from fractions import Fraction

import numpy as np

from conftest import golden_rows
from test_oracle_pins import GRID, exact_nearest_index, f32_exact


def _lone(a):
    x = np.zeros((1, 32), np.float32)
    x[0, 5] = a
    return x


def test_page_rule_golden(oracle_lib):
    for row in golden_rows("oas_page_rule.txt"):
        a, s0, bits, nf = row.split()
        for mode, want in (("ocp", s0), ("oas_bits", bits), ("oas_nf", nf)):
            _, s = oracle_lib.quantize(_lone(float(a)), mode)
            assert int(s[0, 0]) == int(want), (a, mode)
    x = _lone(6.5)
    x[0, 10:13] = 0.5
    _, s = oracle_lib.quantize(x, "oas_nf")
    assert int(s[0, 0]) == 127


def exact_no_overflow_byte(amax: Fraction) -> int:
    s = 0
    while s < 252 and amax / Fraction(2) ** (s - 127) > 6:
        s += 1
    return s


def test_bits_rule_exact_rational(oracle_lib):
    """Random block maxima over the whole range, the page's rule evaluated on
    exact rationals (no-overflow scale, then the (3, 3.5] test)."""
    rng = np.random.default_rng(31)
    m = rng.uniform(1, 2, 4000)
    m[:200] = rng.choice([1.5, 1.75, 1.625, 1.875, 1.0], 200)  # range edges
    e = rng.integers(-140, 128, 4000)
    a = np.ldexp(m, e).astype(np.float32)
    a = a[np.isfinite(a) & (a > 0)]
    x = np.zeros((a.size, 32), np.float32)
    x[:, 0] = a
    x[:, 1] = a * np.float32(0.3)
    _, s = oracle_lib.quantize(x, "oas_bits")
    for i, v in enumerate(a):
        amax = f32_exact(v)
        snf = exact_no_overflow_byte(amax)
        vn = amax / Fraction(2) ** (snf - 127)
        want = snf - 1 if (snf >= 1 and 3 < vn <= Fraction(7, 2)) else snf
        assert int(s[i, 0]) == want, (v, snf, float(vn))


def test_page_modes_never_exceed_252(oracle_lib):
    big = np.float32(np.finfo(np.float32).max)
    for a in (big, np.float32(7.9) * np.float32(2.0 ** 125), np.float32(6.5) * np.float32(2.0 ** 125)):
        for mode in ("oas_bits", "oas_nf"):
            c, s = oracle_lib.quantize(_lone(a), mode)
            assert int(s[0, 0]) <= 252
            assert np.isfinite(oracle_lib.dequantize(c, s, "f32")).all()


def test_nf_decision_vs_exact_rational(oracle_lib):
    """The pinned fp32 decision of oas_nf equals the exact-arithmetic decision
    wherever the exact gap exceeds fp32 rounding; both outcomes occur."""
    rng = np.random.default_rng(32)
    picked_low = kept = 0
    for _ in range(500):
        x = (rng.integers(-16, 17, 32) / 8.0).astype(np.float32)
        x[: rng.integers(0, 24)] = rng.choice([0.5, 0.25, 0.75, 1.5, 0.0], 1)[0]
        x[rng.integers(32)] = rng.choice([6.25, 6.5, 7.0, 7.5, 5.0, 4.0, -6.75])
        x *= np.float32(2.0 ** rng.integers(-30, 30))
        _, s = oracle_lib.quantize(x[None], "oas_nf")
        amax = max(abs(f32_exact(v)) for v in x)
        snf = exact_no_overflow_byte(amax)

        def sse(b):
            X = Fraction(2) ** (b - 127)
            return sum((abs(f32_exact(v)) - GRID[exact_nearest_index(abs(f32_exact(v)) / X)] * X) ** 2
                       for v in x)
        e0, e1 = sse(snf), sse(snf - 1)
        if abs(e0 - e1) > Fraction(1, 2 ** 16) * max(e0, e1):
            want = snf - 1 if e1 < e0 else snf
            assert int(s[0, 0]) == want
            picked_low += want == snf - 1
            kept += want == snf
    assert picked_low >= 5 and kept >= 5


def test_qsnr_closed_form(oracle_lib):
    # a lone 5 (scale 1) decodes to 4: SSE = 1, sum x^2 = 25, QSNR = 10 log10 25
    x = _lone(5.0)
    c, s = oracle_lib.quantize(x)
    _, sse, ssq = oracle_lib.block_mse(x, c, s, with_energy=True)
    assert sse == 1.0 and ssq == 25.0
    assert abs(oracle_lib.qsnr_db(x, c, s) - 10 * math.log10(25.0)) < 1e-12


def test_modes_error_ordering(oracle_lib):
    """Where a mode chooses by error among candidates, its block SSE is never
    above the SSE at the candidate it would otherwise keep."""
    import workloads
    x = workloads.to_bf16_bits(workloads.bf16_laplace_sparse_outliers(seed=9, shape=(32, 4096)))
    c0, s0 = oracle_lib.quantize(x, "ocp")
    b0, _ = oracle_lib.block_mse(x, c0, s0)
    for mode in ("oas", "oas_nf", "oas_bits"):
        c, s = oracle_lib.quantize(x, mode)
        b, _ = oracle_lib.block_mse(x, c, s)
        assert np.isfinite(b).all()
        d = s.astype(int) - s0.astype(int)
        assert set(np.unique(d)) <= {-1, 0, 1}
    c, s = oracle_lib.quantize(x, "oas")
    b, _ = oracle_lib.block_mse(x, c, s)
    assert (b <= b0 * (1 + 1e-6)).all()
