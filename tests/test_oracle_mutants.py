"""Plant mistakes in copies of the oracle and check that its pins catch each one.

Every mutant is a one-line edit of ``oracle/gemm_oracle.c`` of the kind a
careless implementation would make (a wrong sign, a dropped term, a swapped
index, an operand read transposed, an off-by-one bound, truncation instead of
rounding).  Each is compiled on the CPU into a temporary library, and the pin
suite is run against it in a child process; the pins must fail.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "sum_sign": ("double p = a * x;\n            s = s + p;", "double p = a * x;\n            s = s - p;"),
    "a_transposed": ("offset(P->oA, i, k, P->lda)", "offset(P->oA, k, i, P->lda)"),
    "b_transposed": ("offset(P->oB, k, j, P->ldb)", "offset(P->oB, j, k, P->ldb)"),
    "beta_dropped": ("r = r + P->beta * c0;\n        d = d + fabs(P->beta) * fabs(c0);\n    }\n    if (P->bias",
                     "r = r + c0;\n        d = d + fabs(P->beta) * fabs(c0);\n    }\n    if (P->bias"),
    "alpha_dropped": ("double r = P->alpha * s;\n    double d = fabs(P->alpha) * t;\n    if (P->beta != 0.0) {\n        double c0",
                      "double r = s;\n    double d = fabs(P->alpha) * t;\n    if (P->beta != 0.0) {\n        double c0"),
    "den_beta_dropped": ("d = d + fabs(P->beta) * fabs(c0);\n    }\n    if (P->bias",
                         "d = d;\n    }\n    if (P->bias"),
    "last_k_dropped": ("k < P->K; ++k) {\n            double a", "k + 1 < P->K; ++k) {\n            double a"),
    "col_major_ignored": ("order == ORC_ROW ? r * ld + c : c * ld + r",
                          "order == ORC_ROW ? r * ld + c : r * ld + c"),
    "batch_stride_b_wrong": ("b0 = b * P->sB", "b0 = b * P->sA"),
    "f16_exponent_off": ("e - 25); /* (1 + m/1024)", "e - 24); /* (1 + m/1024)"),
    "round_truncates": ("nearbyint(x / q)", "trunc(x / q)"),
    "no_overflow_to_inf": ("if (fabs(r) > maxfinite) r = copysign(INFINITY, x);", ""),
    "subnormal_spacing": ("if (e < emin) e = emin;", ""),
    "flat_index_wrong": ("i = (e / N) % M, j = e % N", "i = (e / N) % M, j = (e + 1) % N"),
    "bias_per_row": ("b * P->sBias + j", "b * P->sBias + i"),
    "bias_batch_stride_dropped": ("b * P->sBias + j", "j"),
    "bias_dropped": ("r = r + bj;", "r = r;"),
    "den_bias_dropped": ("d = d + fabs(bj);", "d = d;"),
    "relu_keeps_negatives": ("r = r > 0.0 ? r : 0.0;", "r = r > 0.0 ? r : -r;"),
    "gelu_tanh_form": ("r = r * 0.5 * (1.0 + erf(r / sqrt(2.0)));",
                       "r = r * 0.5 * (1.0 + tanh(0.7978845608 * (r + 0.044715 * r * r * r)));"),
    "gelu_wrong_scale": ("erf(r / sqrt(2.0))", "erf(r / 2.0)"),
    "e4m3_bias_off": ("e - 10); /* (1 + m/8)", "e - 9); /* (1 + m/8)"),
    "e4m3_nan_rule": ("if (e == 15 && m == 7)", "if (e == 15)"),
    "e5m2_subnormal_scale": ("ldexp((double)m, -16)", "ldexp((double)m, -15)"),
    "e5m2_inf_as_nan": ("v = m ? NAN : INFINITY;\n    else if (e == 0)\n        v = ldexp((double)m, -16);",
                        "v = NAN;\n    else if (e == 0)\n        v = ldexp((double)m, -16);"),
    "b_type_ignored": ("load(P->b_type, P->B", "load(P->in_type, P->B"),
    # the same mistakes in the row-blocked full-matrix path
    "rows_sum_sign": ("sr[j] = sr[j] + p;", "sr[j] = sr[j] - p;"),
    "rows_den_not_abs": ("tr[j] = tr[j] + fabs(p);", "tr[j] = tr[j] + p;"),
    "rows_a_transposed": ("offset(oA, i0 + r, k, lda)", "offset(oA, k, i0 + r, lda)"),
    "rows_b_transposed": ("offset(oB, k, j, ldb)", "offset(oB, j, k, ldb)"),
    "rows_b_type_ignored": ("load(b_type, B,", "load(in_type, B,"),
    "rows_batch_b_decoded_once": ("if (b == 0 || sB != 0)", "if (b == 0)"),
    # 8-bit outputs (saturating rounding)
    "f8out_no_saturation": ("double r = a > maxfinite ? maxfinite : round_to_format",
                            "double r = a > maxfinite ? a : round_to_format"),
    "f8out_e4m3_max_480": ("const double maxfinite = e5m2 ? 57344.0 : 448.0;",
                           "const double maxfinite = e5m2 ? 57344.0 : 480.0;"),
    "f8out_subnormal_scale": ("return sign | (uint8_t)ldexp(r, -(emin - p + 1));",
                              "return sign | (uint8_t)ldexp(r, -(emin - p));"),
    "f8out_e5m2_bias": ("bias = e5m2 ? 15 : 7;", "bias = e5m2 ? 16 : 7;"),
    # block-scaled (MX) inputs
    "mx_scale_block_16": ("i * P->ldsa + k / 32]", "i * P->ldsa + k / 16]"),
    "mx_b_scale_row_of_a": ("j * P->ldsb + k / 32]", "i * P->ldsb + k / 32]"),
    "mx_b_uses_lda": ("j * P->ldb + k)", "j * P->lda + k)"),
    "mx_stream_high_bits_first": ("v = (v >> (bit % 8)) & ((1u << w) - 1);",
                                  "v = (v >> ((8 - w - bit % 8) & 7)) & ((1u << w) - 1);"),
    "mx_e3m2_bias_off": ("decode_small(bits & 0x3f, 3, 2, 3)", "decode_small(bits & 0x3f, 3, 2, 2)"),
    "mx_subnormal_exponent": ("ldexp((double)m, 1 - bias - mbits)", "ldexp((double)m, -bias - mbits)"),
    "mx_e8m0_bias_128": ("ldexp(1.0, (int)bits - 127)", "ldexp(1.0, (int)bits - 128)"),
    "mx_e8m0_nan_ignored": ("bits == 255 ? NAN :", "0 ? NAN :"),
    "mx_sum_sign": ("const double p = xa * xb;\n            s = s + p;",
                    "const double p = xa * xb;\n            s = s - p;"),
    "mx_beta_dropped": ("r = r + P->beta * c0;\n        d = d + fabs(P->beta) * fabs(c0);\n    }\n    *ref = r;",
                        "r = r + c0;\n        d = d + fabs(P->beta) * fabs(c0);\n    }\n    *ref = r;"),
    "mx_alpha_dropped": ("double r = P->alpha * s;\n    double d = fabs(P->alpha) * t;\n    if (P->beta != 0.0) {\n        const double c0",
                         "double r = s;\n    double d = fabs(P->alpha) * t;\n    if (P->beta != 0.0) {\n        const double c0"),
    "mx_last_k_dropped": ("k < P->K; ++k) {\n            const double xa", "k + 1 < P->K; ++k) {\n            const double xa"),
    "mx_scale_raw_exponent": ("decode_e8m0(P->SB[", "(double)(P->SB["),
    "rows_last_k_dropped": ("for (int64_t k = 0; k < K; ++k) {\n                    const double *x",
                            "for (int64_t k = 0; k + 1 < K; ++k) {\n                    const double *x"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut_src = tmp_path / "mutant.c"
    mut_src.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    obuild.build(src=str(mut_src), out=lib)
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
