"""Planted mistakes in copies of the oracle must be caught by the pins.

Each case copies oracle/oracle.c, applies one textual mutation (a dropped
term, a flipped sign, a transposed or mis-indexed operand, a wrong exponent
bias, a lost scale, ...), compiles the copy into a temporary directory with
the host compiler, and runs every pin against it: at least one pin must fail.
The real oracle is never modified.  No GPU needed."""
import os

import pytest

import oracle
from tests import oracle_pins

pytestmark = pytest.mark.timeout(600)

MUTATIONS = {
    "transposed_B": ("J->B16[k * J->b_rs + j * J->b_cs]", "J->B16[j * J->b_rs + k * J->b_cs]"),
    "dropped_last_k": ("for (int64_t k = 0; k < J->K; ++k)", "for (int64_t k = 0; k + 1 < J->K; ++k)"),
    "flipped_sign": ("        s += x * y;", "        s -= x * y;"),
    "a_uses_row_stride_twice": ("J->A16[i * J->a_rs + k * J->a_cs]", "J->A16[i * J->a_rs + k * J->a_rs]"),
    "bf16_shift": ("(uint32_t)h << 16", "(uint32_t)h << 15"),
    "e4m3_bias": ("ldexp(8.0 + (double)m, e - 10)", "ldexp(8.0 + (double)m, e - 9)"),
    "e4m3_subnormal": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "e4m3_no_nan": ("if (e == 0xF && m == 0x7) return NAN;", ""),
    "e4m3_sign_lost": ("return sign ? -mag : mag;", "return mag;"),
    "e8m0_bias": ("ldexp(1.0, (int)e - 127)", "ldexp(1.0, (int)e - 128)"),
    "mx_scale_B_lost": ("s += sa * sb * inner;", "s += sa * inner;"),
    "mx_block_index_lost": ("J->SA[i * J->sa_ld + b]", "J->SA[i * J->sa_ld]"),
    "mx_transposed_B": ("J->B8[k * J->b_rs + j * J->b_cs]", "J->B8[j * J->b_rs + k * J->b_cs]"),
    "mx_block_width": ("k < 32 * b + 32; ++k", "k < 32 * b + 31; ++k"),
    # the sampled MX entry point (the checker of every at-size MX comparison)
    "mx_sample_swapped": ("mx_element(J, J->rows[t], J->cols[t], &c, &a);",
                          "mx_element(J, J->cols[t], J->rows[t], &c, &a);"),
    "mx_sample_col_from_row": ("mx_element(J, J->rows[t], J->cols[t], &c, &a);",
                               "mx_element(J, J->rows[t], J->rows[t], &c, &a);"),
    "mx_sample_abs_is_value": ("        mx_element(J, J->rows[t], J->cols[t], &c, &a);\n        J->out[t] = c;\n"
                               "        if (J->absout) J->absout[t] = a;",
                               "        mx_element(J, J->rows[t], J->cols[t], &c, &a);\n        J->out[t] = c;\n"
                               "        if (J->absout) J->absout[t] = c;"),
    "abs_product_signed": ("        m += fabs(x) * fabs(y);\n    }\n    *c = s;",
                           "        m += x * y;\n    }\n    *c = s;"),
    "rowloop_sign": ("crow[j] += x * y;", "crow[j] -= x * y;"),
    "rowloop_wrong_row": ("const uint16_t* brow = J->B16 + k * J->b_rs;",
                          "const uint16_t* brow = J->B16 + (k / 2) * J->b_rs;"),
    "rowloop_abs_signed": ("arow[j] += fabs(x) * fabs(y);", "arow[j] += x * y;"),
    "ledger_stages_fixed": ("int64_t smem = stages * hbm;", "int64_t smem = 2 * hbm;"),
    "ledger_flops_single": ("int64_t flops = 2 * m * n * k;", "int64_t flops = m * n * k;"),
    "ledger_fits_strict": ("out[3] = smem <= smem_limit ? 1 : 0;", "out[3] = smem < smem_limit ? 1 : 0;"),
    # attention (part IV of the MLSys book summary)
    "attn_scale_dropped": ("s[j] = J->scale * dot;", "s[j] = dot;"),
    "attn_causal_top_left": ("int64_t last = i + (J->Sk - J->Sq);", "int64_t last = i;"),
    "attn_causal_strict": ("nkeys = last + 1 < J->Sk ? last + 1 : J->Sk;",
                           "nkeys = last < J->Sk ? last : J->Sk;"),
    "attn_no_max_shift": ("s[j] = exp(s[j] - mx);", "s[j] = exp(s[j]);"),
    "attn_gqa_modulo": ("const int64_t hk = h / g;", "const int64_t hk = h % J->Hkv;"),
    "attn_v_from_k": ("const uint16_t* v = vb + j * J->vs[2];", "const uint16_t* v = kb + j * J->ks[2];"),
    "attn_lse_no_log": ("*lse = mx + log(l);", "*lse = mx + l;"),
    "attn_not_normalised": ("        o[d] /= l;\n", ""),
    "attn_omag_signed": ("omag[d] += s[j] * fabs(x);", "omag[d] += s[j] * x;"),
    "attn_dim_stride_lost": ("oracle_bf16_value(q[d * J->qs[3]])", "oracle_bf16_value(q[d])"),
    "attn_dropped_last_d": ("for (int64_t d = 0; d < J->D; ++d)\n            dot +=",
                            "for (int64_t d = 0; d + 1 < J->D; ++d)\n            dot +="),
    "attn_first_key_dropped": ("o[d] += s[j] * x;", "o[d] += j ? s[j] * x : 0.0;"),
    "attn_empty_rows_nan": ("    if (nkeys == 0) {\n        *lse = -INFINITY;\n        return;\n    }\n", ""),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found in oracle.c"
    mutated = tmp_path / "oracle_mutated.c"
    mutated.write_text(src.replace(old, new))  # every occurrence
    lib = oracle.build(str(mutated), str(tmp_path / f"liboracle_{name}.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, OverflowError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
