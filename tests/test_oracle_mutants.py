"""The oracle's pins catch plausible mistakes (no GPU).

Each case copies oracle/oracle.c, plants one mistake (a swapped nibble, a
wrong bias, a dropped scale or term, a transposed index, a wrong sign, a
window offset lost), builds the copy with gcc into a temporary library and runs
the pin tests of test_oracle_pins.py against it: at least one pin must fail.
The real oracle is never modified.
"""
from __future__ import annotations

import os
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("q4_nibbles_swapped", "w[j] = (float)(d * (double)(lo - 8));\n      w[j + 16] = (float)(d * (double)(hi - 8));",
     "w[j] = (float)(d * (double)(hi - 8));\n      w[j + 16] = (float)(d * (double)(lo - 8));"),
    ("q4_offset_7", "w[j] = (float)(d * (double)(lo - 8));", "w[j] = (float)(d * (double)(lo - 7));"),
    ("q8_unsigned_codes", "(double)(int8_t)b[2 + j]", "(double)b[2 + j]"),
    ("q8_scale_dropped", "w[j] = (float)(d * (double)(int8_t)b[2 + j]);", "w[j] = (float)((double)(int8_t)b[2 + j]);"),
    ("fp16_subnormal_exponent", "ldexp((double)man, -24)", "ldexp((double)man, -25)"),
    ("fp16_bias", "ldexp((double)(1024 + man), exp - 25)", "ldexp((double)(1024 + man), exp - 24)"),
    ("fp16_sign_dropped", "return sign ? -v : v;", "return v;"),
    ("e8m0_bias_128", "return ldexp(1.0, e - 127);", "return ldexp(1.0, e - 128);"),
    ("e8m0_255_finite", "if (e == 255) return NAN;", "if (e == 256) return NAN;"),
    ("e2m1_subnormal", "double v = (e == 0) ? 0.5 * m", "double v = (e == 0) ? 1.0 * m"),
    ("e2m1_sign_bit", "int s = (code >> 3) & 1;", "int s = (code >> 2) & 1;"),
    ("mxfp4_scale_last", "double s = e8m0_value(b[0]);", "double s = e8m0_value(b[16]);"),
    ("x_transposed", "(double)x[b * qk + j]", "(double)x[j * nb + b]"),
    ("last_block_dropped", "for (int64_t b = 0; b < nb; ++b) {\n    decode_block(fmt, row + b * bb, w);",
     "for (int64_t b = 0; b + 1 < nb; ++b) {\n    decode_block(fmt, row + b * bb, w);"),
    ("window_offset_lost", "gemv_row(j->fmt, j->w + r * j->rb", "gemv_row(j->fmt, j->w + (r - j->r0) * j->rb"),
    ("abs_sum_signed", "aacc += fabs(p);", "aacc += p;"),
    ("silu_sign", "h[i] = g[i] / (1.0 + exp(-g[i])) * u[i];", "h[i] = g[i] / (1.0 + exp(g[i])) * u[i];"),
    ("rms_mean_dropped", "1.0 / sqrt(ss / (double)n + eps)", "1.0 / sqrt(ss + eps)"),
    ("gelu_scale", "erfc(-v[i] / sqrt(2.0))", "erfc(-v[i])"),
    ("gelu_cancelling", "0.5 * v[i] * erfc(-v[i] / sqrt(2.0))", "0.5 * v[i] * (1.0 + erf(v[i] / sqrt(2.0)))"),
    ("q4k_min_added", "w[32 * j + l] = (float)(d * sc[j] * q - dmin * m[j]);",
     "w[32 * j + l] = (float)(d * sc[j] * q + dmin * m[j]);"),
    ("q4k_dmin_is_d", "double dmin = orc_half_to_double((uint16_t)(b[2] | (b[3] << 8)));",
     "double dmin = orc_half_to_double((uint16_t)(b[0] | (b[1] << 8)));"),
    ("q4k_scale_min_swapped", "sc[j] = s[j] & 63;\n    m[j] = s[j + 4] & 63;",
     "sc[j] = s[j + 4] & 63;\n    m[j] = s[j] & 63;"),
    ("q4k_top_bits_wrong_byte", "sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);",
     "sc[j] = (s[j + 4] & 15) | ((s[j] >> 6) << 4);"),
    ("q4k_nibble_parity", "int q = (j % 2 == 0) ? (byte & 15) : (byte >> 4);",
     "int q = (j % 2 == 1) ? (byte & 15) : (byte >> 4);"),
    ("q4k_code_stride", "int byte = qs[32 * (j / 2) + l];", "int byte = qs[32 * (j % 4) + l];"),
    ("q6k_offset_31", "w[e] = (float)(d * scale[e / 16] * (q - 32));", "w[e] = (float)(d * scale[e / 16] * (q - 31));"),
    ("q6k_scale_per_32", "w[e] = (float)(d * scale[e / 16] * (q - 32));", "w[e] = (float)(d * scale[e / 32] * (q - 32));"),
    ("q6k_high_shift", "int high = (qh[32 * h + l] >> (2 * i)) & 3;", "int high = (qh[32 * h + l] >> i) & 3;"),
    ("q6k_low_select", "int low = (ql[64 * h + 32 * (i % 2) + l] >> (4 * (i / 2))) & 15;",
     "int low = (ql[64 * h + 32 * (i / 2) + l] >> (4 * (i % 2))) & 15;"),
    ("q6k_d_first", "double d = orc_half_to_double((uint16_t)(b[208] | (b[209] << 8)));",
     "double d = orc_half_to_double((uint16_t)(b[0] | (b[1] << 8)));"),
    ("q6k_unsigned_scale", "const int8_t *scale = (const int8_t *)(b + 192);", "const uint8_t *scale = b + 192;"),
    ("kquant_block_weights_32", "return (fmt == ORC_Q4_K || fmt == ORC_Q6_K) ? 256 : 32;", "return 32;"),
    ("combine_stride_dropped", "acc += w[s] * y[s * y_stride + i];", "acc += w[s] * y[i];"),
    ("combine_weight_index", "acc += w[s] * y[s * y_stride + i];", "acc += w[0] * y[s * y_stride + i];"),
]

# pins, cheapest first; a mutant is caught at the first one that fails
PINS = [
    pins.test_block_sizes_match_pages,
    pins.test_q8_0_hand_built_blocks,
    pins.test_q4_0_hand_built_block,
    pins.test_e8m0_golden_points,
    pins.test_mxfp4_every_scale_and_code_against_published_tables,
    pins.test_layout_is_row_major_out_by_in,
    pins.test_closed_forms,
    pins.test_windows_equal_slices_of_the_whole,
    pins.test_gemv_against_exact_rationals,
    pins.test_silu_mul_against_scipy_expit,
    pins.test_rms_carry_closed_forms,
    pins.test_q4_0_every_code_at_every_position,
    pins.test_fp16_all_65536_patterns_match_struct,
    pins.test_q8_0_bruteforce_every_scale_and_code,
    pins.test_q4_k_field_order_and_formula,
    pins.test_q4_k_scale_field_is_a_bijection,
    pins.test_q4_k_codes_are_a_bijection,
    pins.test_q4_k_hand_built_blocks,
    pins.test_q6_k_codes_are_a_bijection_and_centered,
    pins.test_q6_k_scales_cover_runs_of_16,
    pins.test_q6_k_hand_built_blocks,
    pins.test_combine_against_exact_rationals_and_special_cases,
]

PARAMS = {
    pins.test_windows_equal_slices_of_the_whole: [dict(fmt=f) for f in (1, 2, 3)],
    pins.test_gemv_against_exact_rationals: [dict(fmt=f, k=64) for f in (1, 2, 3)],
}


def _caught(lib) -> str | None:
    saved = oracle._lib
    oracle._lib = lib
    try:
        for pin in PINS:
            for kw in PARAMS.get(pin, [dict()]):
                try:
                    pin(**kw)
                except (AssertionError, ValueError):
                    return pin.__name__
        return None
    finally:
        oracle._lib = saved


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mutant.c")
        so = os.path.join(d, "libmutant.so")
        open(c, "w").write(src.replace(old, new))
        oracle.build(src=c, out=so)
        lib = oracle.load(so)
        caught_by = _caught(lib)
    assert caught_by is not None, f"no pin caught mutant {name}"


def test_unmutated_copy_passes_every_pin():
    with tempfile.TemporaryDirectory() as d:
        so = os.path.join(d, "libcopy.so")
        oracle.build(src=SRC, out=so)
        assert _caught(oracle.load(so)) is None
