"""Plant plausible mistakes in copies of the oracle's C source (on the CPU)
and require that the pins catch every one of them."""
import os
import tempfile

import pytest

import oracle
import pins

# (name, exact text in csa_oracle.c, replacement)
MUTANTS = [
    ("e2m1_bias", "ldexp(1.0 + m / 2.0, e - 1)", "ldexp(1.0 + m / 2.0, e)"),
    ("e2m1_subnormal", "ldexp((double)m, -1)", "ldexp((double)m, 0)"),
    ("nibble_order", "(i % 2 == 0) ? (byte & 15) : (byte >> 4)", "(i % 2 == 0) ? (byte >> 4) : (byte & 15)"),
    ("idx_scale_block", "r[64 + i / 32]", "r[64 + (i / 32 + 1) % 4]"),
    ("idx_stride", "rows + j * IDX_ROW;\n    for (int i = 0; i < 128", "rows + j * 64;\n    for (int i = 0; i < 128"),
    ("e4m3_subnormal", "ldexp(m / 8.0, -6)", "ldexp(m / 8.0, -7)"),
    ("e4m3_bias", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("e4m3_nan", "if (e == 15 && m == 7) return NAN;", ""),
    ("ue8m0_bias", "ldexp(1.0, byte - 127)", "ldexp(1.0, byte - 128)"),
    ("ue8m0_nan", "if (byte == 255) return NAN;", ""),
    ("kv_scale_block", "r[576 + i / 64]", "r[576 + (i / 64 + 1) % 7]"),
    ("f16_endian", "r[448 + 2 * t] | (r[448 + 2 * t + 1] << 8)", "(r[448 + 2 * t] << 8) | r[448 + 2 * t + 1]"),
    ("f16_bias", "ldexp(1.0 + m / 1024.0, e - 15)", "ldexp(1.0 + m / 1024.0, e - 14)"),
    ("f16_subnormal", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("rope_dropped", "out[j * 512 + 448 + t] = (float)csa_oracle_f16(bits);", "out[j * 512 + 448 + t] = 0.0f * bits;"),
    ("score_no_relu", "double relu = (d > 0.0) ? d : 0.0;", "double relu = d;"),
    ("score_no_weight", "s += (double)w_idx[h] * relu;", "s += relu;"),
    ("score_q_transposed", "(double)q_idx[h * 128 + i]", "(double)q_idx[i * n_idx_heads + h]"),
    ("score_float_accum", "double d = 0.0;\n      for (int i = 0; i < 128; ++i) d +=",
     "float d = 0.0f;\n      for (int i = 0; i < 128; ++i) d +="),
    ("topk_ascending", "if (a->s > b->s) return -1;", "if (a->s > b->s) return 1;"),
    ("topk_tie_high_index", "return (a->j < b->j) ? -1 : (a->j > b->j) ? 1 : 0;",
     "return (a->j > b->j) ? -1 : (a->j < b->j) ? 1 : 0;"),
    ("topk_nan_first", "if (an != bn) return an ? 1 : -1;", "if (an != bn) return an ? -1 : 1;"),
    ("attn_no_scale", "logit[t] = softmax_scale * d;", "logit[t] = d;"),
    ("attn_lse_no_max", "lse[h] = (float)(m + log(z));", "lse[h] = (float)log(z);"),
    ("attn_no_normalise", "(float)(acc[e] / z)", "(float)(acc[e])"),
    ("attn_q_row", "const float *q = q_attn + (size_t)h * 512;", "const float *q = q_attn;"),
    ("step_k_not_k_eff", "sel, (int)k_eff, q_attn, n_heads", "sel, k, q_attn, n_heads"),
    ("step_heads_swapped", "csa_oracle_score(idx_rows, n_rows, q_idx, w_idx, n_idx_heads, scores);",
     "csa_oracle_score(idx_rows, n_rows, q_idx, w_idx, n_heads, scores);"),
    ("step_attends_first_rows", "int64_t k_eff = csa_oracle_topk(scores, n_rows, k, sel, sel_score);",
     "int64_t k_eff = csa_oracle_topk(scores, n_rows, k, sel, sel_score);\n  for (int64_t i = 0; i < k_eff; ++i) sel[i] = (int32_t)i;"),
    ("step_scale_dropped", "q_attn, n_heads, softmax_scale, out,\n                              lse);",
     "q_attn, n_heads, 1.0, out,\n                              lse);"),
    ("dense_skips_last_row", "csa_oracle_attention(kv_rows, n_rows, all, (int)n_rows,",
     "csa_oracle_attention(kv_rows, n_rows, all, (int)n_rows - (n_rows > 1),"),
    ("dense_row_offset", "for (int64_t j = 0; j < n_rows; ++j) all[j] = (int32_t)j;",
     "for (int64_t j = 0; j < n_rows; ++j) all[j] = (int32_t)(j / 2);"),
    ("pack_e4m3_emax", "int sb = pack_scale_byte(amax, 8);", "int sb = pack_scale_byte(amax, 7);"),
    ("pack_e2m1_emax", "int sb = pack_scale_byte(amax, 2);", "int sb = pack_scale_byte(amax, 3);"),
    ("pack_tie_odd", "if (isnan(v)) continue;\n    double d = fabs(a - v);\n    if (d < best_d || (d == best_d && (c & 1) == 0))",
     "if (isnan(v)) continue;\n    double d = fabs(a - v);\n    if (d < best_d || (d == best_d && (c & 1) == 1))"),
    ("pack_f16_tie_odd", "double v = csa_oracle_f16(c);\n    double d = fabs(a - v);\n    if (d < best_d || (d == best_d && (c & 1) == 0))",
     "double v = csa_oracle_f16(c);\n    double d = fabs(a - v);\n    if (d < best_d || (d == best_d && (c & 1) == 1))"),
    ("pack_negative_zero", "r[64 * b + i] = (uint8_t)((c != 0 && signbit(y)) ? (c | 0x80) : c);",
     "r[64 * b + i] = (uint8_t)(signbit(y) ? (c | 0x80) : c);"),
    ("pack_zero_block_byte", "if (amax == 0.0) return 127;\n  int e;\n  frexp(amax, &e); /* floor(log2 amax) = e - 1 */\n  int b =",
     "if (amax == 0.0) return 0;\n  int e;\n  frexp(amax, &e); /* floor(log2 amax) = e - 1 */\n  int b ="),
    ("pack_f16_overflow", "if (a >= 65520.0) return s | 0x7C00;", "if (a >= 65536.0) return s | 0x7C00;"),
    ("pack_f16_sign", "  return s | best; /* the sign is kept, -0 included (IEEE) */", "  return best;"),
    ("pack_rope_bytes", "r[448 + 2 * t] = (uint8_t)(h & 0xFF);\n      r[448 + 2 * t + 1] = (uint8_t)(h >> 8);",
     "r[448 + 2 * t] = (uint8_t)(h >> 8);\n      r[448 + 2 * t + 1] = (uint8_t)(h & 0xFF);"),
    ("merge_weights_swapped", "(wa * out_a[h * 512 + e] + wb * out_b[h * 512 + e])", "(wb * out_a[h * 512 + e] + wa * out_b[h * 512 + e])"),
    ("merge_lse_no_max", "lse[h] = (float)(M + log(wa + wb));", "lse[h] = (float)log(wa + wb);"),
    ("multi_token_query_stride", "q_idx + (size_t)t * n_idx_heads * 128, w_idx + (size_t)t * n_idx_heads,",
     "q_idx + (size_t)t * 128, w_idx + (size_t)t * n_idx_heads,"),
    ("multi_token_output_order", "sel + (size_t)t * k, sel_score ? sel_score + (size_t)t * k : NULL",
     "sel + (size_t)(n_tokens - 1 - t) * k, sel_score ? sel_score + (size_t)(n_tokens - 1 - t) * k : NULL"),
    ("q4_scale_offset", "shared = (e - 1) - 2;", "shared = (e - 1) - 1;"),
    ("q4_ceil_log2", "shared = (e - 1) - 2;", "shared = e - 2;"),
    ("q4_tie_odd", "double d = fabs(a - csa_oracle_e2m1(c));\n    if (d < best_d || (d == best_d && (c & 1) == 0))",
     "double d = fabs(a - csa_oracle_e2m1(c));\n    if (d < best_d || (d == best_d && (c & 1) == 1))"),
    ("q4_tie_to_lower", "double d = fabs(a - csa_oracle_e2m1(c));\n    if (d < best_d || (d == best_d && (c & 1) == 0))",
     "double d = fabs(a - csa_oracle_e2m1(c));\n    if (d < best_d || (0))"),
    ("q4_sign_dropped", "return signbit(y) ? (best | 8) : best;", "return (y < 0.0) ? (best | 8) : best;"),
    ("q4_no_clamp", "if (shared < -127) shared = -127;", ""),
    ("q4_zero_block_byte", "int shared = -127; /* the all-zero block */", "int shared = 0; /* the all-zero block */"),
    ("q4_nibble_order", "-shared));\n    }\n    for (int i = 0; i < 64; ++i) r[i] = (uint8_t)(code[2 * i] | (code[2 * i + 1] << 4));",
     "-shared));\n    }\n    for (int i = 0; i < 64; ++i) r[i] = (uint8_t)((code[2 * i] << 4) | code[2 * i + 1]);"),
    ("pack_idx_nibble_order", "(c | 8) : c;\n      }\n    }\n    for (int i = 0; i < 64; ++i) r[i] = (uint8_t)(code[2 * i] | (code[2 * i + 1] << 4));",
     "(c | 8) : c;\n      }\n    }\n    for (int i = 0; i < 64; ++i) r[i] = (uint8_t)((code[2 * i] << 4) | code[2 * i + 1]);"),
    ("q4_scale_slot", "r[64 + b] = (uint8_t)(shared + 127);", "r[64 + (b + 1) % 4] = (uint8_t)(shared + 127);"),
]


def _caught(o) -> list:
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(o)
        except AssertionError:
            failed.append(check.__name__)
        except (ValueError, FloatingPointError, MemoryError):
            failed.append(check.__name__)
    return failed


def test_mutant_list_applies():
    src = open(oracle.SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, f"mutant {name}: pattern must occur exactly once"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mut.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        so = oracle.build(src=path, out=os.path.join(d, "libmut.so"))
        failed = _caught(oracle.Oracle(so))
    assert failed, f"planted mistake '{name}' passed every pin"
