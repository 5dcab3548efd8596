// csa_bound.hpp -- the rigorous bracket of a filter score.
//
// The filter (csa_score.hpp) computes s~_j from a query held to 3 fp6 terms
// with fp32 matrix-core sums.  The exact score the selection orders by is
// S_j = fl32(s_j), s_j = sum_h w_h max(0, q_h . k_j) evaluated in fp64 (as
// the reference does).  For every row
//     |s~_j - S_j| <= beta_j = sum_b Z_b 2^(s_jb - 127) + Z_abs,
// s_jb the row's UE8M0 byte of block b, with per-query constants
//     Z_b   = 6 (1 + 2^-10) sum_h |w_h| (rho_hb + 2^-15 A_hb),
//     Z_abs = 2^-117 sum_h |w_h|,
// where rho_hb and A_hb are the L1 norms over block b of head h of the query
// residual and of the terms plus residual (QFragNorms).  Why this holds:
//   * |k_ji| <= 6 * 2^(s_jb - 127) (E2M1's largest magnitude is 6), so the
//     residual contributes at most sum_h |w_h| sum_b rho_hb 6 2^(s_jb-127)
//     (the ReLU is 1-Lipschitz);
//   * each of the 3 chained matrix-core products sums 128 exact products and
//     the accumulator in fp32: at most 3 * 130 roundings of 2^-24 relative
//     to the sum of magnitudes (any summation order), plus at most 2^-126
//     per step if the unit flushes fp32 subnormals (the 2^-117 term);
//   * the epilogue (16 fused multiply-adds and 4 additions per row) and the
//     final fp32 rounding of the exact score add 21 more roundings;
//   * the fp64 evaluation of the reference adds below 2^-44 relative;
// 412 * 2^-24 < 2^-15 covers all the relative terms; (1 + 2^-10) covers the
// rounding of Z's own evaluation.  A block byte of 253 or more can decode
// to an fp32 infinity: such a row gets an infinite bracket, as does a row
// whose filter score is not finite.  The bracket is then rounded outward to
// fp32: u = roundup(s~ + beta), l = rounddown(s~ - beta).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

struct FilterBound {
  double z[4];  // Z_b (including the factor 6 (1 + 2^-10))
  double zabs;  // Z_abs
};

// The next fp32 value above / below f (f not NaN).
__device__ __forceinline__ float f32_next_up(float f) {
  if (f == __builtin_inff()) return f;
  if (f == 0.0f) return __uint_as_float(1u);  // smallest subnormal
  const uint32_t b = __float_as_uint(f);
  return __uint_as_float((b >> 31) ? b - 1u : b + 1u);
}
__device__ __forceinline__ float f32_next_down(float f) { return -f32_next_up(-f); }

// fp64 -> fp32 rounded toward +inf / -inf.
__device__ __forceinline__ float f32_round_up(double x) {
  const float f = (float)x;
  return (double)f < x ? f32_next_up(f) : f;
}
__device__ __forceinline__ float f32_round_down(double x) {
  const float f = (float)x;
  return (double)f > x ? f32_next_down(f) : f;
}

// 2^(e - 127) as fp64 for a scale byte e <= 252 (always a normal fp64).
__device__ __forceinline__ double pow2_ue8m0(uint32_t e) {
  return __longlong_as_double((long long)((uint64_t)(e + 896u) << 52));
}

// Bracket [lo, up] of the exact score of a row with filter score st and
// block scale bytes sb (byte b = block b); returns its half-width beta (with
// the outward margins; +inf for an infinite bracket).
__device__ __forceinline__ double row_bracket(float st, uint32_t sb, const FilterBound &B, float &up, float &lo) {
  bool inf = !(fabsf(st) <= 3.40282347e38f);
  double beta = B.zabs;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t e = (sb >> (8 * b)) & 255u;
    inf = inf || e >= 253u;
    beta += B.z[b] * pow2_ue8m0(e < 253u ? e : 0u);
  }
  if (inf) {
    up = __builtin_inff();
    lo = -__builtin_inff();
    return __builtin_inf();
  }
  // outward margin for the fp64 evaluation of beta and of st +- beta
  const double s = (double)st;
  beta = beta * (1.0 + 0x1p-30) + fabs(s) * 0x1p-50;
  up = f32_round_up(s + beta);
  lo = f32_round_down(s - beta);
  return beta;
}

}  // namespace csa
