"""Planted mistakes in the oracle must trip at least one pin.

Each case copies ``oracle/oracle.c``, applies one textual change of the kind a
slip would make (a dropped term, a wrong sign or index, swapped operands, a
reversed bit order, truncation instead of rounding), builds the copy with gcc
into a temporary directory and runs every pin against it. All of this happens
on the CPU; the shipped oracle is untouched.
"""

import os

import pytest

import oracle
from tests import pins

MUTANTS = {
    "msb_first_codes": ("(word >> (bits * pos))", "(word >> (bits * ((int)per_word - 1 - pos)))"),
    "word_index_mod": ("row_words[k / per_word]", "row_words[k % per_word]"),
    "narrow_code_mask": ("(1u << bits) - 1u", "(1u << (bits - 1)) - 1u"),
    "scale_bias_swapped": (
        "oracle_bf16_to_f64(row_scales[g]) * q + oracle_bf16_to_f64(row_biases[g])",
        "oracle_bf16_to_f64(row_biases[g]) * q + oracle_bf16_to_f64(row_scales[g])"),
    "bias_dropped": (
        "oracle_bf16_to_f64(row_scales[g]) * q + oracle_bf16_to_f64(row_biases[g])",
        "oracle_bf16_to_f64(row_scales[g]) * q"),
    "bias_subtracted": (
        "oracle_bf16_to_f64(row_scales[g]) * q + oracle_bf16_to_f64(row_biases[g])",
        "oracle_bf16_to_f64(row_scales[g]) * q - oracle_bf16_to_f64(row_biases[g])"),
    "group_of_128": ("int64_t g = k / group;", "int64_t g = k / (2 * group);"),
    "first_k_dropped": ("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 1; k < K; ++k)"),
    "sign_flipped": ("    acc += oracle_bf16_to_f64(x_row[k])", "    acc -= oracle_bf16_to_f64(x_row[k])"),
    "x_row_zero_only": ("p->x + t * p->K", "p->x + (t % 1) * p->K"),
    "expert_ignored": ("const uint32_t* w_row = p->w + (e * p->N + n) * words;",
                       "const uint32_t* w_row = p->w + (n) * words;"),
    "expert_scales_ignored": ("const uint16_t* s_row = p->s + (e * p->N + n) * groups;",
                              "const uint16_t* s_row = p->s + (n) * groups;"),
    "invalid_rows_use_expert_0": ("if (e < 0 || e >= p->E) return 0.0;",
                                  "if (e < 0 || e >= p->E) e = 0;"),
    "output_transposed": ("      r = i / p->N;\n      n = i % p->N;",
                          "      r = i % p->rows;\n      n = i / p->rows;"),
    "bf16_truncates": ("double r = nearbyint(ldexp(a, 8 - e));", "double r = floor(ldexp(a, 8 - e));"),
    "bf16_ties_away": ("double r = nearbyint(ldexp(a, 8 - e));", "double r = round(ldexp(a, 8 - e));"),
    "token_ignored": ("return dot_row(p->x + t * p->K,", "return dot_row(p->x + r * p->K,"),
    "invalid_token_kept": ("if (t < 0 || t >= p->T) return 0.0;", "if (t < 0 || t >= p->T) t = 0;"),
    "dense_layout_swapped": ("uint16_t wv = p->layout == 0 ? we[n * p->K + k] : we[k * p->N + n];",
                             "uint16_t wv = p->layout == 1 ? we[n * p->K + k] : we[k * p->N + n];"),
    "dense_expert_ignored": ("const uint16_t* we = p->w + e * p->N * p->K;", "const uint16_t* we = p->w;"),
    "dense_token_ignored": ("const uint16_t* x_row = p->x + p->K * t;",
                            "const uint16_t* x_row = p->x + p->K * r;"),
    "dense_invalid_rows_use_expert_0": ("if (e < 0 || p->E <= e) return 0.0;",
                                        "if (e < 0 || p->E <= e) e = 0;"),
    "dense_invalid_token_kept": ("if (t < 0 || p->T <= t) return 0.0;", "if (t < 0 || p->T <= t) t = 0;"),
    "dense_first_k_dropped": ("  for (int64_t k = 0; k < p->K; ++k) {", "  for (int64_t k = 1; k < p->K; ++k) {"),
    "dense_f16_read_as_bf16": ("return dtype == 0 ? oracle_bf16_to_f64(h) : oracle_f16_to_f64(h);",
                               "return oracle_bf16_to_f64(h);"),
    "f16_exponent_bias": ("v = ldexp((double)(1024 + frac), field - 25);",
                          "v = ldexp((double)(1024 + frac), field - 24);"),
    "f16_implicit_one_dropped": ("v = ldexp((double)(1024 + frac), field - 25);",
                                 "v = ldexp((double)(frac), field - 25);"),
    "f16_subnormal_scale": ("v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    "f16_truncates": ("double r = nearbyint(ldexp(a, 11 - e));", "double r = floor(ldexp(a, 11 - e));"),
    "f16_no_overflow": ("if (biased >= 31) return (uint16_t)(sign | 0x7C00u);",
                        "if (biased >= 32) return (uint16_t)(sign | 0x7C00u);"),
    "bf16_no_overflow": ("if (biased >= 255) return (uint16_t)(sign | 0x7F80u);",
                         "if (biased >= 256) return (uint16_t)(sign | 0x7F80u);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC_PATH).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(force=True, src=str(path), out=str(tmp_path / "liboracle_mutant.so"))
    O = oracle.Oracle(lib)
    failures = []
    for check in pins.ALL_CHECKS:
        try:
            check(O)
        except AssertionError:
            failures.append(check.__name__)
    assert failures, f"no pin caught the planted mistake {name}"


def test_unmutated_copy_passes(tmp_path):
    """The harness itself: an unmodified copy passes every pin."""
    path = tmp_path / "oracle_copy.c"
    path.write_text(open(oracle.SRC_PATH).read())
    O = oracle.Oracle(oracle.build(force=True, src=str(path), out=str(tmp_path / "lib.so")))
    for check in pins.ALL_CHECKS:
        check(O)
    assert os.path.exists(oracle.SRC_PATH)
