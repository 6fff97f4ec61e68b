"""The oracle's pins catch plausible mistakes in it.

Each case below plants one mistake in a private copy of the oracle's C
source (a wrong bias, a tie broken the wrong way, a dropped term, a swapped
nibble, a strict compare made loose, an accumulation order changed ...),
builds that copy and runs the CPU pins of the oracle against it. At least one
pin must fail on every mutant, and every pin must pass on the unchanged
oracle. The mistakes are planted on the CPU only: no GPU code is involved.
"""
import importlib.util
import inspect
import os
import shutil
import warnings

import numpy as np
import pytest

import test_oracle_mbs
import test_oracle_mxfp8
import test_oracle_nvfp4
import test_oracle_oas_order as order
import test_oracle_page_modes
import test_oracle_pins
import workloads
from conftest import ROOT

ORACLE_DIR = os.path.join(ROOT, "oracle")

# (name, text in mxref.c that occurs exactly once, replacement)
MUTANTS = [
    # E8M0 shared scale ("MXFP8: Block-32 scaling" and the MX format table:
    # scale = 2^(floor(log2 amax) - emax of the element type), emax = 2)
    ("ocp_bias_off_by_one", "int s = floor_log2 - 2 + 127;", "int s = floor_log2 - 1 + 127;"),
    ("ocp_clamp_to_255",
     "int s = floor_log2 - 2 + 127;\n  if (s < 0) s = 0;\n  if (s > 254) s = 254;",
     "int s = floor_log2 - 2 + 127;\n  if (s < 0) s = 0;\n  if (s > 255) s = 255;"),
    ("ocp_no_low_clamp",
     "int s = floor_log2 - 2 + 127;\n  if (s < 0) s = 0;",
     "int s = floor_log2 - 2 + 127;"),
    ("nonfinite_misses_inf", "if (isnan(xb[i]) || isinf(xb[i])) return 255;",
     "if (isnan(xb[i])) return 255;"),
    # E2M1 element encode: nearest, ties to even, saturating at 6
    ("ties_away_from_zero", "      idx = (lo % 2 == 0) ? lo : hi;", "      idx = hi;"),
    ("ties_to_odd", "      idx = (lo % 2 == 0) ? lo : hi;", "      idx = (lo % 2 == 0) ? hi : lo;"),
    ("ties_toward_zero", "      idx = (lo % 2 == 0) ? lo : hi;", "      idx = lo;"),
    ("saturate_from_4", "  if (v >= 6.0) {\n    idx = 7;", "  if (v >= 4.0) {\n    idx = 7;"),
    ("grid_value_3_as_2_5", "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}",
     "{0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 4.0, 6.0}"),
    ("negative_zero_loses_sign", "int sign = signbit(x) ? 8 : 0;", "int sign = (x < 0) ? 8 : 0;"),
    ("encode_scale_off_by_one", "double v = fabs(x) / ldexp(1.0, s - 127); /* exact",
     "double v = fabs(x) / ldexp(1.0, s - 126); /* exact"),
    # decode
    ("decode_drops_sign", "  return (c & 8) ? -mag : mag;\n}\n\n/* Block squared",
     "  return mag;\n}\n\n/* Block squared"),
    ("decode_255_as_inf", "  if (s == 255) return NAN;\n  double mag = kGrid",
     "  if (s == 255) return INFINITY;\n  double mag = kGrid"),
    # packing: even element in the low nibble
    ("pack_nibbles_swapped", "(uint8_t)(code[2 * t] | (code[2 * t + 1] << 4));",
     "(uint8_t)(code[2 * t + 1] | (code[2 * t] << 4));"),
    ("unpack_nibbles_swapped",
     "int c = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);\n          double q = mxref_decode(c, s);",
     "int c = (i % 2 == 0) ? (byte >> 4) : (byte & 0xF);\n          double q = mxref_decode(c, s);"),
    # overflow-aware scale ("Unveiling the Potential of Quantization with
    # MXFP4", technical summary section 2.A) and its pinned fp32 error
    ("oas_tie_takes_smaller", "if (sse_low < sse_ocp)", "if (sse_low <= sse_ocp)"),
    ("oas_candidate_above", "mxref_oas_sse32(xb, s0 - 1, s0);", "mxref_oas_sse32(xb, s0 + 1, s0);"),
    ("oas_units_of_the_candidate", "const double unit = ldexp(1.0, 127 - h);",
     "const double unit = ldexp(1.0, 127 - c);"),
    ("sse_one_accumulator", "acc_odd = fmaf(d1, d1, acc_odd);", "acc_even = fmaf(d1, d1, acc_even);"),
    ("sse_unfused", "acc_even = fmaf(d0, d0, acc_even);", "acc_even = acc_even + d0 * d0;"),
    ("sse_sequential_groups", "return (grp[0] + grp[1]) + (grp[2] + grp[3]);",
     "return ((grp[0] + grp[1]) + grp[2]) + grp[3];"),
    ("sse_drops_a_group", "return (grp[0] + grp[1]) + (grp[2] + grp[3]);",
     "return (grp[0] + grp[1]) + grp[2];"),
    ("bits_rule_open_at_3_5", "v > 3.0 && v <= 3.5", "v > 3.0 && v < 3.5"),
    ("bits_rule_without_low_clamp", "if (snf >= 1 && v > 3.0", "if (v > 3.0"),
    ("nf_tie_takes_smaller", "if (sse_low < sse_nf)", "if (sse_low <= sse_nf)"),
    ("no_overflow_bound_inclusive", "amax / ldexp(1.0, s - 127) > 6.0) s++;",
     "amax / ldexp(1.0, s - 127) >= 6.0) s++;"),
    ("no_overflow_clamp_254", "while (s < 252 && amax", "while (s < 254 && amax"),
    # block error and tensor sums
    ("mse_error_sign", "double d = xv - qf;", "double d = xv + qf;"),
    ("mse_divides_by_16", "(float)(sse / BLOCK);", "(float)(sse / 16);"),
    ("mse_reconstruction_not_rounded", "double qf = isnan(q) ? q : (double)(float)q;",
     "double qf = q;"),
    ("energy_drops_an_element", "ssq += xv * xv;", "ssq += xv * xv * (i % 32 != 31);"),
    ("sse_drops_an_element", "sse += d * d;", "sse += d * d * (i % 32 != 5);"),
    ("oas_skipped_at_byte_1", "if (mode == MXREF_OAS && s0 >= 1)", "if (mode == MXREF_OAS && s0 >= 2)"),
    ("nf_skipped_at_byte_1", "  if (snf >= 1) {\n    float sse_nf", "  if (snf >= 2) {\n    float sse_nf"),
    ("tensor_sse_in_fp32", "j->sse += (long double)sse;", "j->sse += (long double)(float)sse;"),
    ("decode_scale_off_by_one", "double mag = kGrid[c & 7] * ldexp(1.0, s - 127);",
     "double mag = kGrid[c & 7] * ldexp(1.0, s - 128);"),
    # element stores
    ("bf16_ties_away", "return (uint16_t)((u + 0x7FFFu + lsb) >> 16);", "return (uint16_t)((u + 0x8000u) >> 16);"),
    ("negative_canonical_nan", "uint32_t q = 0x7FC00000u; /* canonical quiet NaN */",
     "uint32_t q = 0xFFC00000u; /* canonical quiet NaN */"),
    # MXFP8 (E4M3 elements, emax 8)
    ("mxfp8_bias_off_by_one", "int s = (e2 - 1) - 8 + 127;", "int s = (e2 - 1) - 7 + 127;"),
    ("mxfp8_saturates_to_nan", "if (v >= 448.0) return sign | 0x7E;", "if (v >= 448.0) return sign | 0x7F;"),
    ("mxfp8_subnormal_scale", "if (e == 0) return ldexp((double)m / 8.0, -6);",
     "if (e == 0) return ldexp((double)m / 8.0, -7);"),
    ("mxfp8_ties_up", "    c = (lo % 2 == 0) ? lo : hi;\n  return sign | c;", "    c = hi;\n  return sign | c;"),
    ("mxfp8_nan_code_decoded", "if (s == 255 || (c & 0x7F) == 0x7F) return NAN;", "if (s == 255) return NAN;"),
    # NVFP4 comparator
    ("nvfp4_tensor_bound_inclusive", "ldexp(amax, t) > 2688.0) t--;", "ldexp(amax, t) >= 2688.0) t--;"),
    ("nvfp4_block_over_4", "float q6 = (float)ab / 6.0f;", "float q6 = (float)ab / 4.0f;"),
    ("nvfp4_decode_scale_sign_lost", "if (block_scale & 0x80) v = -v;", "if (block_scale & 0x100) v = -v;"),
    ("nvfp4_scale_saturates_to_nan", "  if (v >= 448.0) return 0x7E;\n  int lo = 0;\n  while",
     "  if (v >= 448.0) return 0x7F;\n  int lo = 0;\n  while"),
    ("nvfp4_negative_zero_loses_sign", "code[i] = (signbit(xb[i]) ? 8 : 0) | (e2m1_code(fabsf(v)) & 7);",
     "code[i] = (xb[i] < 0 ? 8 : 0) | (e2m1_code(fabsf(v)) & 7);"),
    ("nvfp4_block_ties_up", "  if (v > mid) return hi;\n  return (lo % 2 == 0) ? lo : hi;\n}\n\nint mxrefnv",
     "  if (v > mid) return hi;\n  return hi;\n}\n\nint mxrefnv"),
    # MBS-Static
    ("mbs_mantissa_truncated", "double m = nearbyint(t);", "double m = floor(t);"),
    ("mbs_decode_factor_128", "double f = 1.0 + macro_mant[i / 128] / 256.0;",
     "double f = 1.0 + macro_mant[i / 128] / 128.0;"),
    ("mbs_sub_block_uses_x", "y[i] = (float)v * inv; /* fp32 multiply */",
     "y[i] = (float)v; /* fp32 multiply */"),
    ("mbs_mantissa_not_capped", "  if (m > 255.0) m = 255.0;\n", "\n"),
    ("mbs_sub_block_16_to_32", "codes[(M * 128 + 16 * j) / 2 + t]", "codes[(M * 128 + 16 * j) / 2 + (t ^ 1)]"),
]


def _order_pin(mod):
    """The fixed-order fp32 block error against its exact integer
    re-derivation, and the decisions that follow from it, on a few thousand
    order-sensitive, tie-prone and near-tie blocks (a smaller run of the
    order pin's own check)."""
    sets = (order._order_sensitive_blocks(91, 1000), workloads.oas_tie_prone_blocks(92, 1000),
            order._near_tie_blocks(93, 1000))
    for x in sets:
        res = order._block_job([list(map(float, b)) for b in x])
        _, s_oas = mod.quantize(x, "oas")
        _, s_nf = mod.quantize(x, "oas_nf")
        for i, (row, r) in enumerate(zip(x, res)):
            b = row.astype(np.float64)
            for pair, s in (("oas", s_oas), ("nf", s_nf)):
                h, hi, lo, _, _ = r[pair]
                if hi is None:
                    continue
                assert np.float32(mod.oas_sse32(b, h, h)).tobytes() == np.float32(hi).tobytes()
                assert np.float32(mod.oas_sse32(b, h - 1, h)).tobytes() == np.float32(lo).tobytes()
                assert int(s[i, 0]) == (h - 1 if lo < hi else h)


# slower pins run last, so a mutant caught early costs little
_SLOW = {"test_exhaustive_bf16_all_scales_exact_integer_bruteforce", "test_bits_rule_exact_rational",
         "test_nf_decision_vs_exact_rational", "test_oas_decision_vs_exact_rational", "_order_pin"}


def _battery():
    pins = []
    for m in (test_oracle_pins, test_oracle_page_modes, test_oracle_mxfp8, test_oracle_nvfp4,
              test_oracle_mbs, order):
        for name, fn in inspect.getmembers(m, inspect.isfunction):
            if (name.startswith("test_") and fn.__module__ == m.__name__
                    and list(inspect.signature(fn).parameters) == ["oracle_lib"]):
                pins.append((f"{m.__name__}.{name}", fn))
    pins.append(("_order_pin", _order_pin))
    return sorted(pins, key=lambda p: (p[0].rsplit(".", 1)[-1] in _SLOW, p[0]))


BATTERY = _battery()


def _load_copy(tmp, source, tag):
    d = os.path.join(tmp, "oracle")
    os.makedirs(d)
    for f in ("__init__.py", "mxref.h"):
        shutil.copy(os.path.join(ORACLE_DIR, f), d)
    with open(os.path.join(d, "mxref.c"), "w") as f:
        f.write(source)
    spec = importlib.util.spec_from_file_location(f"oracle_{tag}", os.path.join(d, "__init__.py"),
                                                  submodule_search_locations=[d])
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build(force=True)
    return mod


def _first_failing_pin(mod):
    for name, pin in BATTERY:
        try:
            with warnings.catch_warnings(), np.errstate(all="ignore"):
                warnings.simplefilter("ignore")
                pin(mod)
        except (Exception, pytest.fail.Exception):
            return name
    return None


def _source():
    with open(os.path.join(ORACLE_DIR, "mxref.c")) as f:
        return f.read()


def test_battery_passes_on_the_oracle(tmp_path):
    assert len(BATTERY) >= 50
    assert _first_failing_pin(_load_copy(str(tmp_path), _source(), "unchanged")) is None


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmp_path):
    src = _source()
    assert src.count(old) == 1, f"mutation site of {name} not unique in mxref.c"
    mod = _load_copy(str(tmp_path), src.replace(old, new), name)
    assert _first_failing_pin(mod) is not None, f"no pin catches the mutant {name}"
