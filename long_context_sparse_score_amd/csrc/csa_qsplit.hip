// csa_qsplit.hip -- split the fp32 indexer query into fp6 (E2M3) terms with
// E8M0 block scales, the A operands of the matrix-core scorer (csa_score.hpp).
//
// For each head h and 32-value block b, with r the residual (initially q):
//   E   = smallest exponent with max|r| / 2^E <= 7.5 (E2M3's largest value),
//   q_t = RNE_E2M3(r / 2^E) * 2^E,   r <- r - q_t   (exact in fp32),
// repeated kTerms times.  The block maximum of r shrinks by at least 2^-3.9
// per term, so after 5 terms every element is within 2^-19.6 of the block
// maximum of q; elements below the maximum keep E2M3's relative precision in
// every term.  The fragment of head h, block b becomes MFMA lane 16b + h%16
// of group h/16.  Eight threads share a fragment, four values each: a term
// costs one three-step maximum and three byte stores per thread.
#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "csa_score.hpp"

namespace csa {

// RNE of |y| <= 7.5 onto the E2M3 grid; returns the 5-bit magnitude code
// (exponent field << 3 | mantissa) and writes the represented magnitude.
__device__ __forceinline__ uint32_t e2m3_mag(float a, float *val) {
  if (a < 1.0f) {  // subnormal range, step 1/8 (8/8 is the first normal)
    const float m = rintf(a * 8.0f);
    *val = m * 0.125f;
    return (uint32_t)m;
  }
  int e = (a >= 4.0f) ? 2 : ((a >= 2.0f) ? 1 : 0);
  float m = rintf(ldexpf(a, 3 - e));  // in [8, 16]
  if (m == 16.0f) { e += 1; m = 8.0f; }
  *val = ldexpf(m, e - 3);
  return ((uint32_t)(e + 1) << 3) | ((uint32_t)m - 8u);
}

struct QSplitArgs {
  const float *q[CSA_MAX_SESSIONS];
  const float *w[CSA_MAX_SESSIONS];
  uint32_t *out;  // [session][kQSplitBytes / 4]
  int n_heads;
};

constexpr int kSplitThreads = 256;
constexpr int kSplitSub = 8;                                                   // threads per fragment
constexpr int kSplitBlocks = kMaxGroups * 16 * 4 * kSplitSub / kSplitThreads;  // 8 per session

__global__ void __launch_bounds__(kSplitThreads) q_split_kernel(const QSplitArgs a) {
  const int sess = blockIdx.y;
  const int gt = blockIdx.x * kSplitThreads + threadIdx.x;
  const int frag = gt / kSplitSub, sub = gt % kSplitSub;
  const int h = frag >> 2, blk = frag & 3;
  const int g = h >> 4, lane = (blk << 4) | (h & 15);  // MFMA lane holding this fragment
  uint32_t *out = a.out + (size_t)sess * (kQSplitBytes / 4);
  float r[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (h < a.n_heads) {
    const float *src = a.q[sess] + h * 128 + 32 * blk + 4 * sub;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = src[i];
  }
  uint8_t *bytes = reinterpret_cast<uint8_t *>(out);
#pragma unroll
  for (int t = 0; t < kTerms; ++t) {
    float amax = fmaxf(fmaxf(fabsf(r[0]), fabsf(r[1])), fmaxf(fabsf(r[2]), fabsf(r[3])));
#pragma unroll
    for (int k = 1; k < kSplitSub; k <<= 1) amax = fmaxf(amax, __shfl_xor(amax, k, kSplitSub));
    int sbyte = 127;
    uint32_t word = 0;
    if (amax > 0.0f) {
      int E = ilogbf(amax) - 2;  // amax / 2^E in [4, 8)
      if (ldexpf(amax, -E) > 7.5f) E += 1;
      E = E < -127 ? -127 : (E > 127 ? 127 : E);
      sbyte = E + 127;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = ldexpf(r[i], -E);
        float mag;
        const uint32_t code = e2m3_mag(fminf(fabsf(y), 7.5f), &mag) | (y < 0.0f ? 32u : 0u);
        r[i] -= copysignf(ldexpf(mag, E), y);
        word |= code << (6 * i);
      }
    }
    // this thread's 4 codes are bits [24 sub, 24 sub + 24) of the fragment
    const size_t rec = (size_t)((g * kTerms + t) * 64 + lane) * 8;  // dword index of the record
    uint8_t *dst = bytes + rec * 4 + 3 * sub;
    dst[0] = (uint8_t)word;
    dst[1] = (uint8_t)(word >> 8);
    dst[2] = (uint8_t)(word >> 16);
    if (sub == 0) {
      out[rec + 6] = (uint32_t)sbyte;
      out[rec + 7] = 0u;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < 64) {
    float *wp = reinterpret_cast<float *>(out + kQSplitDwords);
    wp[threadIdx.x] = (threadIdx.x < a.n_heads) ? a.w[sess][threadIdx.x] : 0.0f;
  }
}

hipError_t launch_q_split(const float *const *q, const float *const *w, int n_sessions, int n_heads,
                          uint32_t *out, hipStream_t st) {
  QSplitArgs a;
  for (int i = 0; i < n_sessions; ++i) {
    a.q[i] = q[i];
    a.w[i] = w[i];
  }
  a.out = out;
  a.n_heads = n_heads;
  q_split_kernel<<<dim3(kSplitBlocks, n_sessions), kSplitThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa
