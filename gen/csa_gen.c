/*
 * csa_gen.c -- seeded synthetic inputs for the CSA decode step.
 *
 * This module only *produces* inputs: random numbers and their encoding into
 * the two packed row formats.  It holds none of the decode step's arithmetic
 * (no decode, no score, no selection, no attention) and shares no code with
 * the CPU oracle or the HIP library; both consume the bytes written here.
 *
 * Row formats (DS4X README, "Packed cache ABI"):
 *   indexer row, 68 B : 128 E2M1 codes, two per byte (64 B), then 4 UE8M0
 *                       scales, one per 32-value block.
 *   KV row,     583 B : 448 E4M3 bytes (non-RoPE), 64 little-endian FP16
 *                       RoPE values (128 B), 7 UE8M0 scales, one per
 *                       64-value non-RoPE block.
 * Nibble order: element 2i in the low nibble, 2i+1 in the high nibble.
 *
 * Encoding rule (OCP Microscaling v1.0, used only here): per block the shared
 * exponent is floor(log2(amax)) - emax_elem (emax 2 for E2M1, 8 for E4M3),
 * stored as a biased byte clamped to [0, 254]; elements are divided by the
 * scale, rounded to nearest-even on the element grid and saturated.  An
 * all-zero block stores byte 127 and +0 codes.
 *
 * Random numbers: a counter-based generator.  splitmix64 (Steele, Lea and
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014) is
 * applied twice:  r(seed, stream, i) = sm(seed ^ sm((stream << 48) ^ i)).
 * N(0,1) uses the Box-Muller cosine branch on draws 2i and 2i+1 in double,
 * rounded once to fp32.  U(0,1) uses the top 24 bits of draw i.
 */
#include "csa_gen.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

#define IDX_ROW 68
#define KV_ROW 583

enum { ST_IDX = 0, ST_KV = 1, ST_ROPE = 2, ST_QIDX = 3, ST_W = 4, ST_QATT = 5 };

static uint64_t sm64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

uint64_t csa_gen_u64(uint64_t seed, uint64_t stream, uint64_t i) {
  return sm64(seed ^ sm64((stream << 48) ^ i));
}

float csa_gen_normal(uint64_t seed, uint64_t stream, uint64_t i) {
  uint64_t a = csa_gen_u64(seed, stream, 2 * i);
  uint64_t b = csa_gen_u64(seed, stream, 2 * i + 1);
  double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
  double u2 = (double)(b >> 11) * 0x1.0p-53;         /* [0, 1) */
  double z = sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
  return (float)z;
}

float csa_gen_uniform(uint64_t seed, uint64_t stream, uint64_t i) {
  return (float)((double)(csa_gen_u64(seed, stream, i) >> 40) * 0x1.0p-24);
}

/* ---------------- encoders (generator only) ---------------- */

/* Round-to-nearest-even of |y| onto the E2M1 magnitude grid, saturating at 6.
 * Returns the 3-bit magnitude code (exponent:mantissa). */
static int e2m1_mag_code(double y) {
  static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  if (!(y < 6.0)) return 7;
  int best = 0;
  double bd = fabs(y - grid[0]);
  for (int c = 1; c < 8; ++c) {
    double d = fabs(y - grid[c]);
    if (d < bd || (d == bd && (c & 1) == 0)) { best = c; bd = d; }
  }
  return best;
}

/* Round |y| to a binary float grid with `mb` mantissa bits, minimum normal
 * exponent `emin` (subnormals below), returning the rounded magnitude.  No
 * saturation here.  rint() uses the default round-to-nearest-even mode. */
static double round_grid(double y, int mb, int emin) {
  if (y == 0.0) return 0.0;
  int e;
  frexp(y, &e); /* y = f * 2^e, f in [0.5, 1) -> floor(log2 y) = e - 1 */
  e -= 1;
  if (e < emin) e = emin;
  double q = ldexp(rint(ldexp(y, mb - e)), e - mb);
  return q;
}

static uint8_t e4m3_encode(double x) {
  int s = signbit(x) ? 0x80 : 0;
  double y = fabs(x);
  double q = round_grid(y, 3, -6);
  if (q > 448.0) q = 448.0;
  if (q == 0.0) return (uint8_t)s;
  int e;
  frexp(q, &e);
  e -= 1;
  if (e < -6) { /* subnormal: q = m * 2^-9 */
    int m = (int)ldexp(q, 9);
    return (uint8_t)(s | m);
  }
  int m = (int)(ldexp(q, 3 - e)) - 8; /* q = (1 + m/8) 2^e */
  if (m == 8) { m = 0; e += 1; }
  if (e < -6) { /* subnormal rounded up to the smallest normal */
    e = -6; m = 0;
  }
  return (uint8_t)(s | ((e + 7) << 3) | m);
}

static uint16_t f16_encode(float xf) {
  double x = (double)xf;
  uint16_t s = signbit(x) ? 0x8000 : 0;
  double y = fabs(x);
  if (isnan(x)) return 0x7E00;
  double q = round_grid(y, 10, -14);
  if (q >= 65520.0 || isinf(y)) return (uint16_t)(s | 0x7C00);
  if (q == 0.0) return s;
  int e;
  frexp(q, &e);
  e -= 1;
  if (e < -14) {
    int m = (int)ldexp(q, 24);
    return (uint16_t)(s | m);
  }
  int m = (int)(ldexp(q, 10 - e)) - 1024;
  if (m == 1024) { m = 0; e += 1; }
  if (e > 15) return (uint16_t)(s | 0x7C00);
  return (uint16_t)(s | ((e + 15) << 10) | m);
}

/* OCP MX shared exponent for a block with max magnitude amax. */
static int mx_scale_byte(double amax, int emax_elem) {
  if (amax == 0.0) return 127;
  int e;
  frexp(amax, &e);
  int x = (e - 1) - emax_elem + 127;
  if (x < 0) x = 0;
  if (x > 254) x = 254;
  return x;
}

void csa_gen_pack_idx_row(const float *v, uint8_t *row) {
  memset(row, 0, IDX_ROW);
  for (int b = 0; b < 4; ++b) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
      double a = fabs((double)v[32 * b + i]);
      if (a > amax) amax = a;
    }
    int sb = mx_scale_byte(amax, 2);
    row[64 + b] = (uint8_t)sb;
    for (int i = 0; i < 32; ++i) {
      int el = 32 * b + i;
      double x = (double)v[el];
      double y = ldexp(fabs(x), 127 - sb);
      int code = e2m1_mag_code(y);
      if (signbit(x) && code != 0) code |= 8;
      row[el >> 1] |= (uint8_t)(code << ((el & 1) * 4));
    }
  }
}

void csa_gen_pack_kv_row(const float *v, uint8_t *row) {
  memset(row, 0, KV_ROW);
  for (int b = 0; b < 7; ++b) {
    double amax = 0.0;
    for (int i = 0; i < 64; ++i) {
      double a = fabs((double)v[64 * b + i]);
      if (a > amax) amax = a;
    }
    int sb = mx_scale_byte(amax, 8);
    row[576 + b] = (uint8_t)sb;
    for (int i = 0; i < 64; ++i) {
      int el = 64 * b + i;
      double x = (double)v[el];
      uint8_t c = e4m3_encode(ldexp(x, 127 - sb));
      if (c == 0x80) c = 0; /* keep zeros as +0 */
      row[el] = c;
    }
  }
  for (int t = 0; t < 64; ++t) {
    uint16_t h = f16_encode(v[448 + t]);
    row[448 + 2 * t] = (uint8_t)(h & 0xFF);
    row[448 + 2 * t + 1] = (uint8_t)(h >> 8);
  }
}

uint16_t csa_gen_f16_bits(float x) { return f16_encode(x); }
uint8_t csa_gen_e4m3_bits(double x) { return e4m3_encode(x); }

/* ---------------- session generation ---------------- */

uint64_t csa_gen_seed(int config_id) { return 0x5EEDC5A0ull + (uint64_t)config_id; }

void csa_gen_idx_rows(uint64_t seed, int session, int64_t row0, int64_t n, uint8_t *out) {
  const uint64_t st = (uint64_t)session * 16 + ST_IDX;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    int64_t j = row0 + r;
    float v[128];
    for (int i = 0; i < 128; ++i) v[i] = csa_gen_normal(seed, st, (uint64_t)j * 128 + i);
    csa_gen_pack_idx_row(v, out + r * IDX_ROW);
  }
}

void csa_gen_kv_rows(uint64_t seed, int session, int64_t row0, int64_t n, uint8_t *out) {
  const uint64_t st = (uint64_t)session * 16 + ST_KV;
  const uint64_t sr = (uint64_t)session * 16 + ST_ROPE;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    int64_t j = row0 + r;
    float v[512];
    for (int i = 0; i < 448; ++i) v[i] = csa_gen_normal(seed, st, (uint64_t)j * 448 + i);
    for (int t = 0; t < 64; ++t) v[448 + t] = csa_gen_normal(seed, sr, (uint64_t)j * 64 + t);
    csa_gen_pack_kv_row(v, out + r * KV_ROW);
  }
}

void csa_gen_queries(uint64_t seed, int session, int n_idx_heads, int n_heads, float *q_idx,
                     float *w_idx, float *q_attn) {
  const uint64_t base = (uint64_t)session * 16;
  for (int i = 0; i < n_idx_heads * 128; ++i) q_idx[i] = csa_gen_normal(seed, base + ST_QIDX, (uint64_t)i);
  for (int h = 0; h < n_idx_heads; ++h) w_idx[h] = csa_gen_uniform(seed, base + ST_W, (uint64_t)h);
  for (int i = 0; i < n_heads * 512; ++i) q_attn[i] = csa_gen_normal(seed, base + ST_QATT, (uint64_t)i);
}

uint64_t csa_gen_fnv1a64(const void *p, int64_t n) {
  const uint8_t *b = (const uint8_t *)p;
  uint64_t h = 0xCBF29CE484222325ull;
  for (int64_t i = 0; i < n; ++i) { h ^= b[i]; h *= 0x100000001B3ull; }
  return h;
}
