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
// where rho_hb is the L1 norm over block b of head h of the query residual
// and A_hb an upper bound on the L1 norm of the terms plus the residual
// (QFragNorms).  Why this holds:
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
// rounding of Z's own evaluation (fp64, once per query).  A block byte of 253
// or more can decode to an fp32 infinity: such a row gets an infinite
// bracket, as does a row whose filter score is not finite.
//
// Per row the bracket is evaluated in fp32 and widened so that no rounding
// can cut into it (every step rounds to nearest):
//   * zf_b, zfabs: Z_b, Z_abs rounded up to fp32 (once per query);
//   * t_b = ldexp(zf_b, s_jb - 127) is exact unless it falls below 2^-126
//     (then off by at most 2^-150) and +inf on overflow;
//   * the four additions of the five nonnegative terms lose at most a
//     factor (1 - 2^-24)^4, so sum >= (beta_j - 2^-148)(1 - 2^-24)^4;
//   * beta' = fma(sum, 1 + 2^-20, 2^-139) >= beta_j + 2^-140, since
//     (1 + 2^-20)(1 - 2^-24)^5 > 1 and 2^-139 (1 - 2^-24) > 2^-140 + 2^-148;
//   * u0 = s~ + beta' is off by at most half an ulp of u0, and
//     u = fma(|u0|, 2^-23, u0) lies at least one ulp above u0 when u0 is
//     normal (|u0| 2^-23 is at least that ulp, and the next fp32 value away
//     from u0 in that direction is then at or below the exact result);
//     when u0 is below 2^-126 the half ulp (2^-150) is inside the 2^-140
//     slack of beta'.  So u >= s~ + beta_j >= S_j; likewise
//     l = fma(|l0|, -2^-23, l0) <= S_j with l0 = s~ - beta'.
//   * In the other direction u <= s~ + beta' + 6 ulp(u), which the lower
//     bound rebuilt from u and beta' (row_lower in the tile kernel) allows
//     for.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

struct FilterBound {
  double z[4];  // Z_b (including the factor 6 (1 + 2^-10))
  double zabs;  // Z_abs
};

// The per-row constants in fp32, rounded up.
struct FilterBoundF {
  float z[4];
  float zabs;
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

__device__ __forceinline__ FilterBoundF bound_f32(const FilterBound &B) {
  FilterBoundF F;
#pragma unroll
  for (int b = 0; b < 4; ++b) F.z[b] = f32_round_up(B.z[b]);
  F.zabs = f32_round_up(B.zabs);
  return F;
}

// Bracket of the exact score of a row with filter score st and block scale
// bytes sb (byte b = block b): returns its half-width beta' (+inf for an
// infinite bracket) and the upper bound u; with LOWER also the lower bound
// l.  All fp32 (the margins above).
template <bool LOWER>
__device__ __forceinline__ float row_bracket(float st, uint32_t sb, const FilterBoundF &F, float &up, float &lo) {
  const uint32_t e0 = sb & 255u, e1 = (sb >> 8) & 255u, e2 = (sb >> 16) & 255u, e3 = sb >> 24;
  const bool inf = !(fabsf(st) <= 3.40282347e38f) || e0 > 252u || e1 > 252u || e2 > 252u || e3 > 252u;
  const float t0 = __builtin_ldexpf(F.z[0], (int)e0 - 127), t1 = __builtin_ldexpf(F.z[1], (int)e1 - 127);
  const float t2 = __builtin_ldexpf(F.z[2], (int)e2 - 127), t3 = __builtin_ldexpf(F.z[3], (int)e3 - 127);
  const float sum = ((t0 + t1) + (t2 + t3)) + F.zabs;
  const float beta = __builtin_fmaf(sum, 1.0f + 0x1p-20f, 0x1p-139f);
  const float u0 = st + beta;
  up = inf ? __builtin_inff() : __builtin_fmaf(fabsf(u0), 0x1p-23f, u0);
  if constexpr (LOWER) {
    const float l0 = st - beta;
    lo = inf ? -__builtin_inff() : __builtin_fmaf(fabsf(l0), -0x1p-23f, l0);
  }
  return inf ? __builtin_inff() : beta;
}

}  // namespace csa
