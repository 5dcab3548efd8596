// csa_score.hpp -- the indexer score filter on gfx950 matrix cores.
//
// Score (lightning-indexer form adopted for the library; the DS4X page
// describes the batch-one scorer only as a block-scaled MXFP4 matrix product
// over the 68-byte rows, "Optimization details"):
//     s_j = sum_h w_h * max(0, q_h . k_j)
//
// The packed rows are consumed as they are stored: the 64 E2M1 code bytes of
// a row are the fp4 B operand of V_MFMA_SCALE_F32_16X16X128_F8F6F4 and its
// four UE8M0 bytes are the B block scales (one per 32 values, exactly the
// row's block structure).  The fp32 query cannot be an MX operand, so it is
// split into kTerms fp6 (E2M3) terms with their own E8M0 block scales,
//     q = sum_t qt + r,   |r| <= max(2^-11.9 blockmax|q|, 2^-130) per element,
// and the dot product is the fp32 accumulation of the kTerms exact-product
// MFMAs.  This is a filter: the split also returns, per (head, block)
// fragment, the L1 norms of the residual r and of the terms, from which the
// tile kernel bounds each row's distance to the exact score rigorously; the
// rows the bound cannot place are rescored exactly (csa_refine.hip).  Each
// lane splits its own fragment in registers (split_qfrag).
//
// Lane layout of the 16x16x128 instruction (verified on MI355X): lane l holds
// A row l%16 and B column l%16, for K elements [32*(l/16), 32*(l/16)+32),
// value i of the slice at bit 6i (fp6) or 4i (fp4); its scale byte is byte 0
// of the scale operand; the 16x16 result gives lane l rows 4*(l/16)+v, v<4,
// of column l%16.  With A = 16 query heads and B = 16 history rows, lane l
// therefore loads the 16 code bytes [16*(l/16), +16) and scale byte 64+l/16
// of row l%16.
#pragma once

#include <utility>

#include "csa_device.hpp"

namespace csa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTerms = 3;        // fp6 terms of the query split
constexpr int kMaxGroups = 4;    // 16-head groups (64 indexer heads)
constexpr int kFmtFp6 = 2;       // MFMA operand format codes: E2M3
constexpr int kFmtFp4 = 4;       // E2M1

constexpr int kScaleWords = (kTerms + 3) / 4;  // A scale bytes packed four per register

// Query formats: kQueryFp32 scores the fp32 query through its kTerms fp6
// terms; kQueryMxfp4 first quantizes it to MXFP4 (quantize_qfrag_fp4) and
// scores the quantized query exactly as one fp4 operand.
constexpr int kQueryFp32 = 0;
constexpr int kQueryMxfp4 = 1;
template <int QF>
struct QueryFormat {
  static constexpr int terms = QF == kQueryMxfp4 ? 1 : kTerms;
  static constexpr int fmt = QF == kQueryMxfp4 ? kFmtFp4 : kFmtFp6;
};

template <int G>
struct QFrag {
  v8i a[G][kTerms];
  int scw[G][kScaleWords];  // byte t%4 of word t/4: E8M0 scale of term t
  float w[G][4];
};

// Norms of one lane's fragment after the split: rho = sum |r| (the
// residual's L1 norm) and mag, an upper bound on the L1 norm of the terms
// plus rho (fp64: no overflow for any finite query).
struct QFragNorms {
  float rho;
  double mag;
};

typedef float v16f_q __attribute__((ext_vector_type(16)));
typedef float v32f_q __attribute__((ext_vector_type(32)));
typedef unsigned v6u_q __attribute__((ext_vector_type(6)));

// This lane's query terms, split from its 32 fp32 query values x (head
// 16 g + l%16 of group g, values [32(l/16), +32): the lane's A operand row
// and K slice).  With r the residual (initially the values):
//   E_0 = smallest exponent with max|x| / 2^E <= 7.5 (E2M3's largest
//         value), E_t = max(E_0 - 4t, -126),
//   q_t = RNE_E2M3(r / 2^E_t) * 2^E_t,   r <- r - q_t   (exact in fp32),
// for t < kTerms.  A term's rounding error is at most a quarter of its
// scale (half the 0.5 spacing of E2M3's top binade), which the next term's
// range 7.5 * 2^(E_t - 4) holds without saturating, so no term saturates
// and every subtraction is exact (both operands are multiples of the
// finer of their spacings and the difference is below 2^(E_t - 2)); after
// 3 terms |r| <= 2^-2 * 2^(E_0 - 8) < 2^-11.9 * max|x|, since max|x| >
// 3.75 * 2^E_0 (below 2^-126 the scales stop at 2^-126 and |r| at 2^-130,
// half the finest term spacing).  Returns the bound's inputs: rho = the
// residual's L1 norm, and mag >= sum_t |q_t| + |r| summed over the block,
// from |q_t| <= |r_{t-1}| + |r_t| (r_{-1} = x) and |r_t| <= 2^(E_t - 2):
// mag = sum |x| + sum_t 32 * 2 * 2^(E_t - 2) = sum |x| + sum_t 2^(E_t + 4).
// Heads past the query's heads carry a zero weight (load_qweights), so
// their terms (split from a clamped head) add exact zeros to the score.
// The conversions are gfx950's scaled fp6 instructions (round to nearest
// even, saturating; verified on MI355X): the packing one interleaves its
// two 16-value inputs (even, odd positions), so value i lands at bit 6i,
// the MFMA operand order; the unpacking one returns the exact term values
// for the residual.
__device__ __forceinline__ QFragNorms split_qfrag(QFrag<1> &q, const float (&x)[32]) {
  v16f_q re, ro;
  float amax = 0.0f, sumx = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    re[i] = x[2 * i];
    ro[i] = x[2 * i + 1];
    amax = fmaxf(amax, fmaxf(fabsf(re[i]), fabsf(ro[i])));
    sumx += fabsf(re[i]) + fabsf(ro[i]);
  }
  // amax = m 2^e, m in [1, 2): amax / 2^(e-2) = 4m is in [4, 8), above 7.5
  // when m > 1.875; a zero block keeps scale 2^0 (its codes are zero)
  const uint32_t ab = __float_as_uint(amax);
  int E0 = (int)(ab >> 23) - 129 + ((ab & 0x7FFFFFu) > 0x700000u ? 1 : 0);
  E0 = amax == 0.0f ? 0 : E0;
  E0 = E0 < -126 ? -126 : (E0 > 127 ? 127 : E0);
#pragma unroll
  for (int w = 0; w < kScaleWords; ++w) q.scw[0][w] = 0;
  double mag = (double)sumx;
#pragma unroll
  for (int t = 0; t < kTerms; ++t) {
    const int E = E0 - 4 * t < -126 ? -126 : E0 - 4 * t;
    const float sc = __uint_as_float((uint32_t)(E + 127) << 23);
    const v6u_q c = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(re, ro, sc);
    const v32f_q d = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(c, sc);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      re[i] -= d[2 * i];
      ro[i] -= d[2 * i + 1];
    }
    mag += __longlong_as_double((long long)((uint64_t)(E + 4 + 1023) << 52));  // 2^(E + 4), E >= -126
    q.a[0][t] = v8i{(int)c[0], (int)c[1], (int)c[2], (int)c[3], (int)c[4], (int)c[5], 0, 0};
    q.scw[0][t / 4] |= (E + 127) << (8 * (t % 4));
  }
  float rho = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) rho += fabsf(re[i]) + fabsf(ro[i]);
  return QFragNorms{rho, mag};
}

// E2M1 code of y (the rounding of an MXFP4 conversion): the magnitude code
// of the E2M1 value nearest to |y|, ties to the even code (0 | 0.5 -> 0,
// 0.5 | 1 -> 1, 1 | 1.5 -> 1, 1.5 | 2 -> 2, 2 | 3 -> 2, 3 | 4 -> 4, 4 | 6 -> 4),
// past 6 saturating to 6 (code 7), with y's sign bit as bit 3.
__device__ __forceinline__ uint32_t e2m1_round(float y) {
  const float a = fabsf(y);
  uint32_t c = (a > 0.25f ? 1u : 0u) + (a >= 0.75f ? 1u : 0u) + (a > 1.25f ? 1u : 0u) + (a >= 1.75f ? 1u : 0u) +
               (a > 2.5f ? 1u : 0u) + (a >= 3.5f ? 1u : 0u) + (a > 5.0f ? 1u : 0u);
  return c | ((__float_as_uint(y) >> 31) << 3);
}

// This lane's query fragment (the same 32 values as split_qfrag's) quantized
// to MXFP4 by the OCP MX v1.0 conversion: the block's UE8M0 byte is
// floor(log2 max|x|) - 2 + 127, clamped at 0 (fp32 exponent field minus 2;
// an all-zero block gets 0), and element i is e2m1_round(x_i / 2^(byte-127))
// (the division is an exact power-of-two multiply except where the quotient
// is far below 0.25 and rounds to a signed zero either way).  The codes are
// the single fp4 A operand (value i at bit 4i) and its scale byte; deq gets
// the quantized values (exact in fp32) and the norms are rho = 0 (the
// quantized query is scored exactly) and mag = sum |deq|.
// With a normal scale (byte >= 1) the conversions are gfx950's scaled fp4
// instructions (two values per instruction, the first in the low nibble;
// round to nearest even, saturating at 6, the sign of a zero kept), and the
// decoded values come back from the scaled fp4 -> fp32 conversion; a block
// whose scale is the subnormal 2^-127 takes e2m1_round.
typedef float v2f_q __attribute__((ext_vector_type(2)));
__device__ __forceinline__ QFragNorms quantize_qfrag_fp4(QFrag<1> &q, const float (&x)[32], float (&deq)[32]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const uint32_t ef = __float_as_uint(amax) >> 23;  // amax >= 0: the exponent field
  const uint32_t byte = ef >= 2u ? ef - 2u : 0u;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  float mag = 0.0f;
  if (byte != 0u) {
    const float sc = __uint_as_float(byte << 23);  // 2^(byte - 127), normal
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float *xj = &x[8 * j];
      uint32_t ww = 0u;
      ww = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ww, xj[0], xj[1], sc, 0);
      ww = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ww, xj[2], xj[3], sc, 1);
      ww = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ww, xj[4], xj[5], sc, 2);
      ww = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ww, xj[6], xj[7], sc, 3);
      w[j] = ww;
      const v2f_q d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ww, sc, 0);
      const v2f_q d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ww, sc, 1);
      const v2f_q d2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ww, sc, 2);
      const v2f_q d3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ww, sc, 3);
      const v2f_q dd[4] = {d0, d1, d2, d3};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        deq[8 * j + 2 * k] = dd[k][0];
        deq[8 * j + 2 * k + 1] = dd[k][1];
        mag += fabsf(dd[k][0]) + fabsf(dd[k][1]);
      }
    }
  } else {
    // 2^127 and 2^-127 (the subnormal 0x00400000) as fp32
    const float inv = __uint_as_float(254u << 23);
    const float sc = __uint_as_float(0x00400000u);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t c = e2m1_round(x[i] * inv);
      w[i / 8] |= c << (4 * (i % 8));
      const float v = e2m1_value(c) * sc;
      deq[i] = v;
      mag += fabsf(v);
    }
  }
#pragma unroll
  for (int t = 0; t < kTerms; ++t) q.a[0][t] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  q.a[0][0] = v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < kScaleWords; ++j) q.scw[0][j] = 0;
  q.scw[0][0] = (int)byte;
  return QFragNorms{0.0f, (double)mag};
}

// The weights of the heads whose results lane `lane` holds for group g:
// heads 16 g + 4(l/16) + v, v < 4 (0 past n_heads).
__device__ __forceinline__ void load_qweights(QFrag<1> &q, const float *wh, int n_heads, int g, int lane) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int hw = 16 * g + 4 * (lane >> 4) + v;
    const float x = wh[hw < n_heads ? hw : n_heads - 1];
    q.w[0][v] = hw < n_heads ? x : 0.0f;
  }
}

struct RowOperand {
  uint4 codes;
  int sb;
};

__device__ __forceinline__ v8i as_b(const RowOperand &o) {
  return v8i{(int)o.codes.x, (int)o.codes.y, (int)o.codes.z, (int)o.codes.w, 0, 0, 0, 0};
}

// Term t of every group for NS row operands: c[s][g] += (query term t of
// group g) x (row operand s).  Issued term-major so that NS*G independent
// accumulation chains are in flight; the op_sel immediate picks term t's
// scale byte out of its packed register.
template <int G, int NS, int T, int FA>
__device__ __forceinline__ void mfma_term(const QFrag<G> &q, const v8i (&b)[NS], const int (&sb)[NS],
                                          v4f (&c)[NS][G]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int r = 0; r < NS; ++r)
      c[r][g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q.a[g][T], b[r], c[r][g], FA, kFmtFp4, T % 4,
                                                                  q.scw[g][T / 4], 0, sb[r]);
  }
}

template <int G, int NS, int FA, int... Ts>
__device__ __forceinline__ void mfma_terms(const QFrag<G> &q, const v8i (&b)[NS], const int (&sb)[NS],
                                           v4f (&c)[NS][G], std::integer_sequence<int, Ts...>) {
  (mfma_term<G, NS, Ts, FA>(q, b, sb, c), ...);
}

// The matrix-core products of NS row operands with one 16-head group's
// query (kTerms fp6 terms, or the one fp4 operand of the quantized query):
// c[r] = sum over terms t, in order, of (term t) x (operand r), each operand
// r being this lane's 16 code bytes of row l%16 and its scale byte.  Lane l
// receives heads 4(l/16) + v, v < 4, of row l%16.
template <int NS, int QF = kQueryFp32>
__device__ __forceinline__ void group_dots(const QFrag<1> &q, const RowOperand (&ops)[NS], v4f (&c)[NS][1]) {
  v8i b[NS];
  int sb[NS];
#pragma unroll
  for (int r = 0; r < NS; ++r) {
    b[r] = as_b(ops[r]);
    sb[r] = ops[r].sb;
    c[r][0] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
  mfma_terms<1, NS, QueryFormat<QF>::fmt>(q, b, sb, c, std::make_integer_sequence<int, QueryFormat<QF>::terms>{});
}

// One head group's contribution to the score partials of four operands (64
// rows): p[r] += w_h * max(0, d_h) over the lane's four heads of the group
// (an fma chain over v, continued group after group), d_h = c[r][v].  A NaN
// d, impossible for valid rows, is not zeroed.
__device__ __forceinline__ void group_acc4(const QFrag<1> &q, const v4f (&c)[4][1], float (&p)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      // ReLU as a signed-integer max of the bits: one instruction, and
      // -0 -> +0 (a float max would add an IEEE quieting step)
      const float d = __int_as_float(max(__float_as_int(c[r][0][v]), 0));
      p[r] = __builtin_fmaf(q.w[0][v], d, p[r]);
    }
  }
}

// The four lane-rows of the partials summed by a reduce-scatter: a 32-lane
// swap pairs operands (0, 2) and (1, 3) across the lane halves, a 16-lane
// swap pairs the results across adjacent lane-rows.  Lane l returns the sum
// for row l%16 of operand l/16 (that is, row l of the 64), as
// (lane-row 0 + lane-row 2) + (lane-row 1 + lane-row 3).
// v_permlane32_swap(x, y) -> (x0, x1, y0, y1), (x2, x3, y2, y3) and
// v_permlane16_swap(x, y) -> (x0, y0, x2, y2), (x1, y1, x3, y3) in 16-lane rows.
__device__ __forceinline__ float rows_reduce4(const float (&p)[4]) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
  const float a = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  const float b = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// The score of a row from its two half partials (first + second).
__device__ __forceinline__ float score_finish(float first, float second) {
  const float s = first + second;
  return s == 0.0f ? 0.0f : s;
}

// This lane's operand data for the 16-row tile starting at `row` (rows past
// `n` are clamped to the last row; callers drop their scores).

__device__ __forceinline__ RowOperand load_row_operand(const uint8_t *__restrict__ idx_rows, int64_t row,
                                                       int64_t n, int lane) {
  int64_t r = row + (lane & 15);
  r = r < n ? r : n - 1;
  const uint32_t *p = reinterpret_cast<const uint32_t *>(idx_rows + r * kIdxRowBytes);
  const int g = lane >> 4;
  RowOperand o;
  o.codes = uint4{p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]};
  o.sb = (int)((p[16] >> (8 * g)) & 255u);
  return o;
}

}  // namespace csa
