// csa_device.hpp -- device-side helpers of the gfx950 CSA library: element
// decoding of the packed rows and the sortable selection key.
//
// Element formats (OCP Microscaling v1.0; IEEE 754 binary16) are decoded by
// building the fp32 bit pattern directly, and block scales are applied as an
// exact multiply by 2^(e-127).  Every product is exactly representable in
// fp32 (a 2- or 4-bit significand times a power of two, never below 2^-136),
// except overflow, which gives +-inf.  fp32 denormals must be preserved (the
// library is compiled with -fno-gpu-flush-denormals-to-zero).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

constexpr int kIdxRowBytes = 68;
constexpr int kKvRowBytes = 583;
constexpr int kKvNope = 448;
constexpr int kTopK = 512;

// Workgroup barrier that orders LDS accesses only: the fences are limited
// to the local address space, so the barrier waits for the wave's LDS
// operations (lgkmcnt) but leaves its global loads in flight, unlike
// __syncthreads(), whose workgroup fence also waits for every outstanding
// vector memory operation.  Not for direct-to-LDS loads (those are vector
// memory operations) or for global memory shared between the waves.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// UE8M0 byte -> 2^(e-127) as fp32; e = 0 is the subnormal 2^-127, 0xFF NaN.
__device__ __forceinline__ float ue8m0_scale(uint32_t e) {
  uint32_t bits = (e == 0u) ? 0x00400000u : ((e == 255u) ? 0x7FC00000u : (e << 23));
  return __uint_as_float(bits);
}

// E2M1 4-bit code -> fp32.  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 is
// the sign (code 8 is -0).
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const uint32_t mag = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
  return __uint_as_float(mag | ((c & 8u) << 28));
}

// E4M3 ("FN": bias 7, no infinities, S.1111.111 = NaN) byte -> fp32.  Both
// cases are computed and selected (no branch: decoders sit in unrolled
// gathers whose loads must stay in flight together).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float norm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  const float sub = (float)m * 0x1p-9f;
  const float v = __uint_as_float(__float_as_uint(e ? norm : sub) | ((c & 0x80u) << 24));
  return ((c & 0x7Fu) == 0x7Fu) ? __uint_as_float(0x7FC00000u) : v;
}

// IEEE binary16 bits -> fp32 (exact, subnormals included), branch-free.
__device__ __forceinline__ float f16_value(uint32_t h) {
  const uint32_t s = (h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
  const float sub = __uint_as_float(__float_as_uint((float)m * 0x1p-24f) | s);
  const uint32_t bits = (e == 31u) ? (0x7F800000u | (m << 13)) : (((e + 112u) << 23) | (m << 13));
  const float nrm = __uint_as_float(bits | s);
  return e == 0u ? sub : nrm;
}

// Monotone map of a score to 32 bits: larger score -> larger value, -0 == +0,
// NaN below every number (value 0).
__device__ __forceinline__ uint32_t score_ord(float x) {
  if (x != x) return 0u;
  uint32_t b = __float_as_uint(x);
  if (x == 0.0f) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float ord_score(uint32_t o) {
  if (o == 0u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Selection key: score order, then lower row index first.  Every real key is
// >= 2^31, so 0 serves as "no key".
__device__ __forceinline__ uint64_t make_key(float s, uint32_t row) {
  return ((uint64_t)score_ord(s) << 32) | (uint64_t)(0xFFFFFFFFu - row);
}
__device__ __forceinline__ uint32_t key_row(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }
__device__ __forceinline__ float key_score(uint64_t k) { return ord_score((uint32_t)(k >> 32)); }

}  // namespace csa
