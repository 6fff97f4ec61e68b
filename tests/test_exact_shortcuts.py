"""CPU proofs of the exact shortcuts the kernels take in place of the plain
arithmetic (each one exhaustive over the inputs the kernels can give it).

1. fl32(a / 6) as one product with fl32(1/6) plus one fma residual
   correction: equal to IEEE division for every fp32 a >= 2^-125 (NVFP4 block
   scale a_b / 6, "Unveiling the Potential of Quantization with MXFP4",
   technical summary section 1; MBS-Static macro factor a_M / 6, section
   2.B). Below 2^-125 the quotient is subnormal and the shortcut differs, so
   the kernels divide there.
2. The NVFP4 element factor S / s_b as 2^t * fl32(1 / s_b) from a table of
   reciprocals: equal to fl32(2^t / s_b) for all 126 finite positive E4M3
   block scales s_b and every tensor exponent t the quantizer can produce.
3. Constants built from bit patterns: the MXFP8 saturation limit
   448 * 2^(s-127) as bf16 ((s + 8) << 7 | 0x60) and fp32
   ((s + 8) << 23 | 0x600000) for every scale byte a finite block can get
   (vLLM MXFP8/MXFP4 page, MXFP8 section: E4M3 elements, largest 448), and
   the unit 2^(127-h) of the overflow-aware error ((254 - h) << 23) for
   every candidate byte h that is evaluated.
"""
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def div6_check(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("div6") / "div6_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-o", exe,
                    os.path.join(HERE, "shortcuts", "div6_check.c"), "-lm", "-lpthread"],
                   check=True)
    return exe


def test_div6_shortcut_exact_from_2_pow_minus_125(div6_check):
    threads = str(max(1, min(8, len(os.sched_getaffinity(0)))))
    r = subprocess.run([div6_check, "0x01000000", "0x7F7FFFFF", threads],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
    assert r.stdout.strip() == "checked 2122317824 patterns, 0 differ"


def test_div6_shortcut_not_exact_below_2_pow_minus_125(div6_check):
    """Why the kernels fall back to division for a < 2^-125 (bit patterns
    below 0x01000000)."""
    r = subprocess.run([div6_check, "0x00000001", "0x00FFFFFF", "4"], capture_output=True,
                       text=True)
    assert r.returncode == 1 and " 0 differ" not in r.stdout, r.stdout


def _e4m3_values():
    """The 126 finite positive E4M3 magnitudes (codes 0x01..0x7E) from the
    fields: exponent bias 7, 3 mantissa bits, exponent 0 subnormal."""
    out = []
    for c in range(1, 0x7F):
        e, m = c >> 3, c & 7
        out.append(np.ldexp(m / 8.0, -6) if e == 0 else np.ldexp(1.0 + m / 8.0, e - 7))
    return np.array(out, np.float32)


def test_e4m3_reciprocal_table_identity():
    v = _e4m3_values()
    assert v.size == 126 and v.max() == 448.0 and v.min() == np.float32(2.0 ** -9)
    one = np.float32(1.0)
    rcp = one / v                                    # the table: IEEE fp32 division
    # t of the tensor factor: 2^t * amax <= 6 * 448 with amax up to the
    # largest finite fp32 gives t >= -117; t is capped at 127
    with np.errstate(over="ignore"):
        for t in range(-117, 128):
            s = np.float32(2.0 ** t)
            via_table = rcp * s
            direct = s / v
            assert np.array_equal(via_table.view(np.uint32), direct.view(np.uint32)), t
    # and no 2^t / s_b in that range is subnormal (so scaling commutes with rounding)
    assert np.float32(2.0 ** -117) / np.float32(448.0) >= np.float32(2.0 ** -126)


def test_mxfp8_saturation_limit_patterns():
    # a finite block's E8M0 byte is (exponent field of amax) - 8 <= 246
    for s in range(0, 247):
        want = np.float32(448.0 * 2.0 ** (s - 127))
        f32 = np.array([((s + 8) << 23) | 0x600000], np.uint32).view(np.float32)[0]
        bf16 = np.array([(((s + 8) << 7) | 0x60) << 16], np.uint32).view(np.float32)[0]
        assert f32 == want and bf16 == want, s


def test_overflow_aware_unit_pattern():
    for h in range(1, 253):
        u = np.array([(254 - h) << 23], np.uint32).view(np.float32)[0]
        assert u == np.float32(2.0 ** (127 - h)), h
