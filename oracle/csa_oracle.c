/*
 * csa_oracle.c -- plain, slow, obviously-correct CPU reference for the CSA
 * decode step.  TEST INFRASTRUCTURE ONLY: nothing on the product path may
 * call, link or load this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header or table
 * with the HIP library.
 *
 * What it follows:
 *  - Row formats: DS4X README, "Packed cache ABI".  A KV row is 448 E4M3
 *    bytes, then 64 FP16 RoPE values, then 7 UE8M0 scales (one per 64-value
 *    non-RoPE block; the RoPE tail is unscaled); 583 bytes.  An indexer row is
 *    128 E2M1 values packed two per byte, then 4 UE8M0 scales (one per
 *    32-value block); 68 bytes.  Readings where the page is silent: fields are
 *    contiguous in the listed order; element 2i sits in the low nibble; FP16
 *    is little-endian.
 *  - Element formats: OCP Microscaling Formats v1.0 (E2M1, E4M3 "FN",
 *    UE8M0) and IEEE 754 binary16.  Tables are built here from those
 *    definitions.
 *  - Score: the lightning-indexer form, s_j = sum_h w_h * ReLU(q_h . k_j),
 *    computed in double from the fp32 inputs and the decoded fp32 row, rounded
 *    once to fp32 (the pages never state the score function; this is the
 *    reading adopted for the whole build).
 *  - Selection: exact top-512 by score, float order, lower row index wins a
 *    tie (DS4X README, "Optimization details" and "CSA score/top-512
 *    fusion").  A full sort is used.
 *  - Attention: textbook softmax attention over the selected rows, with the
 *    decoded 512-value row used as both key and value, in double.
 *  - Multi-token score/top-k (DS4X README, "Packed prefill implementation":
 *    batch score/top-k): for each token its own score over the same rows and
 *    its own exact top-k, token after token.
 *  - Dense attention (the HCA layers of DS4X README, "What DS4X changes" and
 *    "Optimization details": exact score-split attention over every
 *    compressed row, no row ceiling): the same textbook softmax attention
 *    over all n rows, each row used once, in row order.
 *  - Packing new rows (the pack path of DS4X README, "Packed cache ABI": new
 *    compressed and raw-ring rows are written in the 583/68-byte formats):
 *    the pages name the formats but not the conversion.  The reading adopted
 *    is the OCP MX v1.0 block conversion: byte = floor(log2 amax) - emax + 127
 *    (emax 8 for E4M3, 2 for E2M1), clamped to [0, 254], 127 for an all-zero
 *    block; each element v / 2^(byte-127) rounded to the nearest element
 *    value, ties to the even significand, saturating (448 for E4M3, 6 for
 *    E2M1); a value that rounds to zero is stored as +0.  The RoPE values are
 *    IEEE binary16, round to nearest even (overflow gives infinity).
 *  - Merging two attention results over disjoint row sets (the sliding-window
 *    raw ring and the compressed rows share one softmax): out = (e^{a-M}
 *    out_a + e^{b-M} out_b) / (e^{a-M} + e^{b-M}), lse = M + log(e^{a-M} +
 *    e^{b-M}), M = max(a, b), a and b the two log-sum-exps, in double.
 *  - MXFP4 query (the block-scaled scorer of DS4X README, "What DS4X
 *    changes" and "Optimization details"): the pages never say how the fp32
 *    query becomes an MXFP4 operand.  The reading adopted is the OCP MX v1.0
 *    conversion of a 32-value block (its section 6.3): shared exponent
 *    floor(log2(max |v|)) - 2, 2 being E2M1's largest exponent, held in UE8M0
 *    (clamped to its range; an all-zero block gets byte 0); each element
 *    v / 2^shared rounded to the nearest E2M1 value, ties to the even
 *    significand, magnitudes past 6 saturating to 6, the sign kept.  The
 *    quantized query is packed exactly like an indexer row, and the
 *    quantized-query score is the score above with the decoded query.
 */
#include "csa_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define IDX_ROW 68
#define KV_ROW 583

/* ---------------- element formats ---------------- */

/* E2M1: sign(1) exponent(2, bias 1) mantissa(1); exponent 0 is subnormal. */
double csa_oracle_e2m1(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? ldexp((double)m, -1) : ldexp(1.0 + m / 2.0, e - 1);
  return s ? -mag : mag;
}

/* E4M3 "FN": sign(1) exponent(4, bias 7) mantissa(3); no infinities,
 * S.1111.111 is NaN; exponent 0 is subnormal. */
double csa_oracle_e4m3(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* UE8M0: unsigned 8-bit exponent, bias 127; 0xFF is NaN. */
double csa_oracle_ue8m0(int byte) {
  if (byte == 255) return NAN;
  return ldexp(1.0, byte - 127);
}

/* IEEE binary16. */
double csa_oracle_f16(int bits) {
  int s = (bits >> 15) & 1, e = (bits >> 10) & 31, m = bits & 1023;
  double mag;
  if (e == 0) mag = ldexp((double)m, -24);
  else if (e == 31) mag = (m == 0) ? INFINITY : NAN;
  else mag = ldexp(1.0 + m / 1024.0, e - 15);
  return s ? -mag : mag;
}

/* ---------------- row decode ---------------- */

void csa_oracle_decode_idx_rows(const uint8_t *rows, int64_t n, float *out) {
  for (int64_t j = 0; j < n; ++j) {
    const uint8_t *r = rows + j * IDX_ROW;
    for (int i = 0; i < 128; ++i) {
      int byte = r[i / 2];
      int code = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
      double scale = csa_oracle_ue8m0(r[64 + i / 32]);
      out[j * 128 + i] = (float)(csa_oracle_e2m1(code) * scale);
    }
  }
}

void csa_oracle_decode_kv_rows(const uint8_t *rows, int64_t n, float *out) {
  for (int64_t j = 0; j < n; ++j) {
    const uint8_t *r = rows + j * KV_ROW;
    for (int i = 0; i < 448; ++i) {
      double scale = csa_oracle_ue8m0(r[576 + i / 64]);
      out[j * 512 + i] = (float)(csa_oracle_e4m3(r[i]) * scale);
    }
    for (int t = 0; t < 64; ++t) {
      int bits = r[448 + 2 * t] | (r[448 + 2 * t + 1] << 8);
      out[j * 512 + 448 + t] = (float)csa_oracle_f16(bits);
    }
  }
}

/* ---------------- indexer score ---------------- */

void csa_oracle_score(const uint8_t *idx_rows, int64_t n, const float *q_idx, const float *w_idx,
                      int n_idx_heads, float *scores) {
  float k[128];
  for (int64_t j = 0; j < n; ++j) {
    csa_oracle_decode_idx_rows(idx_rows + j * IDX_ROW, 1, k);
    double s = 0.0;
    for (int h = 0; h < n_idx_heads; ++h) {
      double d = 0.0;
      for (int i = 0; i < 128; ++i) d += (double)q_idx[h * 128 + i] * (double)k[i];
      double relu = (d > 0.0) ? d : 0.0;
      s += (double)w_idx[h] * relu;
    }
    float f = (float)s;
    if (f == 0.0f) f = 0.0f; /* -0 is stored as +0 */
    scores[j] = f;
  }
}

/* ---------------- exact top-k ---------------- */

typedef struct {
  float s;
  int32_t j;
} pair_t;

/* Larger score first; NaN after every number; equal scores by lower index. */
static int pair_cmp(const void *pa, const void *pb) {
  const pair_t *a = (const pair_t *)pa, *b = (const pair_t *)pb;
  int an = isnan(a->s), bn = isnan(b->s);
  if (an != bn) return an ? 1 : -1;
  if (!an) {
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
  }
  return (a->j < b->j) ? -1 : (a->j > b->j) ? 1 : 0;
}

int64_t csa_oracle_topk(const float *scores, int64_t n, int k, int32_t *sel, float *sel_score) {
  int64_t k_eff = (n < k) ? n : k;
  pair_t *p = (pair_t *)malloc(sizeof(pair_t) * (size_t)(n > 0 ? n : 1));
  if (!p) return -1;
  for (int64_t j = 0; j < n; ++j) {
    p[j].s = scores[j];
    p[j].j = (int32_t)j;
  }
  qsort(p, (size_t)n, sizeof(pair_t), pair_cmp);
  for (int i = 0; i < k; ++i) {
    if (i < k_eff) {
      sel[i] = p[i].j;
      if (sel_score) sel_score[i] = p[i].s;
    } else {
      sel[i] = -1;
      if (sel_score) sel_score[i] = -INFINITY;
    }
  }
  free(p);
  return k_eff;
}

/* ---------------- sparse attention ---------------- */

int csa_oracle_attention(const uint8_t *kv_rows, int64_t n_rows, const int32_t *sel, int n_sel,
                         const float *q_attn, int n_heads, double softmax_scale, float *out,
                         float *lse) {
  if (n_sel == 0) {
    for (int i = 0; i < n_heads * 512; ++i) out[i] = 0.0f;
    if (lse)
      for (int h = 0; h < n_heads; ++h) lse[h] = -INFINITY;
    return 0;
  }
  float *kv = (float *)malloc(sizeof(float) * 512 * (size_t)n_sel);
  double *logit = (double *)malloc(sizeof(double) * (size_t)n_sel);
  double *acc = (double *)malloc(sizeof(double) * 512);
  if (!kv || !logit || !acc) {
    free(kv); free(logit); free(acc);
    return -1;
  }
  for (int t = 0; t < n_sel; ++t) {
    if (sel[t] < 0 || sel[t] >= n_rows) {
      free(kv); free(logit); free(acc);
      return -2;
    }
    csa_oracle_decode_kv_rows(kv_rows + (int64_t)sel[t] * KV_ROW, 1, kv + (size_t)t * 512);
  }
  for (int h = 0; h < n_heads; ++h) {
    const float *q = q_attn + (size_t)h * 512;
    double m = -INFINITY;
    for (int t = 0; t < n_sel; ++t) {
      double d = 0.0;
      for (int e = 0; e < 512; ++e) d += (double)q[e] * (double)kv[(size_t)t * 512 + e];
      logit[t] = softmax_scale * d;
      if (logit[t] > m) m = logit[t];
    }
    double z = 0.0;
    for (int e = 0; e < 512; ++e) acc[e] = 0.0;
    for (int t = 0; t < n_sel; ++t) {
      double p = exp(logit[t] - m);
      z += p;
      for (int e = 0; e < 512; ++e) acc[e] += p * (double)kv[(size_t)t * 512 + e];
    }
    for (int e = 0; e < 512; ++e) out[(size_t)h * 512 + e] = (float)(acc[e] / z);
    if (lse) lse[h] = (float)(m + log(z));
  }
  free(kv); free(logit); free(acc);
  return 0;
}

/* ---------------- multi-token score/top-k ---------------- */

int csa_oracle_score_topk_multi(const uint8_t *idx_rows, int64_t n, const float *q_idx, const float *w_idx,
                                int n_tokens, int n_idx_heads, int k, int32_t *sel, float *sel_score) {
  float *scores = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  if (!scores) return -1;
  for (int t = 0; t < n_tokens; ++t) {
    csa_oracle_score(idx_rows, n, q_idx + (size_t)t * n_idx_heads * 128, w_idx + (size_t)t * n_idx_heads,
                     n_idx_heads, scores);
    if (csa_oracle_topk(scores, n, k, sel + (size_t)t * k, sel_score ? sel_score + (size_t)t * k : NULL) < 0) {
      free(scores);
      return -1;
    }
  }
  free(scores);
  return 0;
}

/* ---------------- dense attention ---------------- */

int csa_oracle_dense_attention(const uint8_t *kv_rows, int64_t n_rows, const float *q_attn, int n_heads,
                               double softmax_scale, float *out, float *lse) {
  int32_t *all = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_rows > 0 ? n_rows : 1));
  if (!all) return -1;
  for (int64_t j = 0; j < n_rows; ++j) all[j] = (int32_t)j;
  int rc = csa_oracle_attention(kv_rows, n_rows, all, (int)n_rows, q_attn, n_heads, softmax_scale, out, lse);
  free(all);
  return rc;
}

/* ---------------- MXFP4 query quantization ---------------- */

/* The E2M1 code nearest to y: the magnitude closest to |y| among the eight
 * E2M1 values (so anything past 6 goes to 6), a tie going to the code with
 * an even significand bit; the sign bit copied from y. */
static int e2m1_nearest(double y) {
  double a = fabs(y);
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c < 8; ++c) {
    double d = fabs(a - csa_oracle_e2m1(c));
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return signbit(y) ? (best | 8) : best;
}

void csa_oracle_quantize_query(const float *q, int n_heads, uint8_t *rows) {
  for (int h = 0; h < n_heads; ++h) {
    uint8_t *r = rows + (int64_t)h * IDX_ROW;
    int code[128];
    for (int b = 0; b < 4; ++b) {
      const float *v = q + (int64_t)h * 128 + 32 * b;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i)
        if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
      int shared = -127; /* the all-zero block */
      if (amax > 0.0) {
        int e;
        frexp(amax, &e); /* amax = f 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
        shared = (e - 1) - 2;
        if (shared < -127) shared = -127;
        if (shared > 127) shared = 127;
      }
      r[64 + b] = (uint8_t)(shared + 127);
      for (int i = 0; i < 32; ++i) code[32 * b + i] = e2m1_nearest(ldexp((double)v[i], -shared));
    }
    for (int i = 0; i < 64; ++i) r[i] = (uint8_t)(code[2 * i] | (code[2 * i + 1] << 4));
  }
}

/* ---------------- packing new rows ---------------- */

/* The element value nearest to |y| among the non-negative values of a
 * format (codes 0..ncodes-1 ascending, value(c) from `val`), a tie going to
 * the code with an even significand bit; values past the largest give the
 * largest (saturation). */
static int nearest_code(double y, int ncodes, double (*val)(int)) {
  double a = fabs(y);
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c < ncodes; ++c) {
    double v = val(c);
    if (isnan(v)) continue;
    double d = fabs(a - v);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return best;
}

/* OCP MX shared-exponent byte of a block with largest magnitude amax. */
static int pack_scale_byte(double amax, int emax_elem) {
  if (amax == 0.0) return 127;
  int e;
  frexp(amax, &e); /* floor(log2 amax) = e - 1 */
  int b = (e - 1) - emax_elem + 127;
  return b < 0 ? 0 : (b > 254 ? 254 : b);
}

/* IEEE binary16 bits of x, round to nearest even: the nearest of the 63,488
 * finite non-negative binary16 values (ties to even), infinity at or beyond
 * 65520 (the midpoint past the largest finite value). */
static int f16_bits_of(double x) {
  int s = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a >= 65520.0) return s | 0x7C00;
  /* candidate neighbours: the binary16 values at the same exponent */
  int best = 0;
  double best_d = INFINITY;
  int e;
  frexp(a, &e);
  int lo = 0, hi = 0x7BFF;
  if (a > 0.0) {
    int ee = (e - 1) + 15; /* biased exponent of a, before rounding */
    if (ee < 1) ee = 0;
    lo = ee > 0 ? ((ee - 1) << 10) : 0;
    hi = (ee + 1) << 10;
    if (hi > 0x7BFF) hi = 0x7BFF;
  } else {
    hi = 0;
  }
  for (int c = lo; c <= hi; ++c) {
    double v = csa_oracle_f16(c);
    double d = fabs(a - v);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return s | best; /* the sign is kept, -0 included (IEEE) */
}

void csa_oracle_pack_kv_rows(const float *v, int64_t n, uint8_t *rows) {
  for (int64_t j = 0; j < n; ++j) {
    const float *x = v + j * 512;
    uint8_t *r = rows + j * KV_ROW;
    for (int b = 0; b < 7; ++b) {
      double amax = 0.0;
      for (int i = 0; i < 64; ++i)
        if (fabs((double)x[64 * b + i]) > amax) amax = fabs((double)x[64 * b + i]);
      int sb = pack_scale_byte(amax, 8);
      r[576 + b] = (uint8_t)sb;
      for (int i = 0; i < 64; ++i) {
        double y = ldexp((double)x[64 * b + i], 127 - sb);
        int c = nearest_code(y, 127, csa_oracle_e4m3); /* codes 0..126: 0 .. 448 */
        r[64 * b + i] = (uint8_t)((c != 0 && signbit(y)) ? (c | 0x80) : c);
      }
    }
    for (int t = 0; t < 64; ++t) {
      int h = f16_bits_of((double)x[448 + t]);
      r[448 + 2 * t] = (uint8_t)(h & 0xFF);
      r[448 + 2 * t + 1] = (uint8_t)(h >> 8);
    }
  }
}

void csa_oracle_pack_idx_rows(const float *v, int64_t n, uint8_t *rows) {
  for (int64_t j = 0; j < n; ++j) {
    const float *x = v + j * 128;
    uint8_t *r = rows + j * IDX_ROW;
    int code[128];
    for (int b = 0; b < 4; ++b) {
      double amax = 0.0;
      for (int i = 0; i < 32; ++i)
        if (fabs((double)x[32 * b + i]) > amax) amax = fabs((double)x[32 * b + i]);
      int sb = pack_scale_byte(amax, 2);
      r[64 + b] = (uint8_t)sb;
      for (int i = 0; i < 32; ++i) {
        double y = ldexp((double)x[32 * b + i], 127 - sb);
        int c = nearest_code(y, 8, csa_oracle_e2m1);
        code[32 * b + i] = (c != 0 && signbit(y)) ? (c | 8) : c;
      }
    }
    for (int i = 0; i < 64; ++i) r[i] = (uint8_t)(code[2 * i] | (code[2 * i + 1] << 4));
  }
}

/* ---------------- merging two attention results ---------------- */

void csa_oracle_lse_merge(const float *out_a, const float *lse_a, const float *out_b, const float *lse_b,
                          int n_heads, float *out, float *lse) {
  for (int h = 0; h < n_heads; ++h) {
    double a = lse_a[h], b = lse_b[h];
    double M = a > b ? a : b;
    if (M == -INFINITY) { /* neither side has a row */
      for (int e = 0; e < 512; ++e) out[h * 512 + e] = 0.0f;
      lse[h] = -INFINITY;
      continue;
    }
    double wa = exp(a - M), wb = exp(b - M);
    for (int e = 0; e < 512; ++e)
      out[h * 512 + e] = (float)((wa * out_a[h * 512 + e] + wb * out_b[h * 512 + e]) / (wa + wb));
    lse[h] = (float)(M + log(wa + wb));
  }
}

/* ---------------- whole decode step ---------------- */

int csa_oracle_decode_step(const uint8_t *idx_rows, const uint8_t *kv_rows, int64_t n_rows,
                           const float *q_idx, const float *w_idx, int n_idx_heads,
                           const float *q_attn, int n_heads, double softmax_scale, int k,
                           int32_t *sel, float *sel_score, float *out, float *lse) {
  float *scores = (float *)malloc(sizeof(float) * (size_t)(n_rows > 0 ? n_rows : 1));
  if (!scores) return -1;
  csa_oracle_score(idx_rows, n_rows, q_idx, w_idx, n_idx_heads, scores);
  int64_t k_eff = csa_oracle_topk(scores, n_rows, k, sel, sel_score);
  free(scores);
  if (k_eff < 0) return -1;
  return csa_oracle_attention(kv_rows, n_rows, sel, (int)k_eff, q_attn, n_heads, softmax_scale, out,
                              lse);
}
