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
//
// The same launch also splits the attention query into three bf16 terms per
// value, stored in the matrix-core operand order of csa_attn.hpp (extra
// workgroups, when an attention query is given).
#include "csa_attn.hpp"
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
  const float *q_attn[CSA_MAX_SESSIONS];
  uint32_t *out;    // [session][kQSplitBytes / 4]
  uint4 *attn_out;  // [session][kAttnQVecs]
  int n_heads;      // indexer heads (0: no indexer split)
  int n_attn_heads;
  int idx_blocks;   // workgroups of the indexer split per session
};

constexpr int kSplitThreads = 256;
constexpr int kSplitSub = 8;                                                   // threads per fragment
constexpr int kSplitBlocks = kMaxGroups * 16 * 4 * kSplitSub / kSplitThreads;  // 8 per session

constexpr int kAttnSplitBlocks = 16 * 4 * 64 / kSplitThreads;  // 16 per session

// Attention query: thread (wave w, step s, lane l) writes the three terms of
// q[16(w%4) + l%16][128(w/4) + 32s + 8(l/16) + i], i < 8.
__device__ void attn_q_split(const QSplitArgs &a, int sess, int t) {
  const int lane = t % 64, s = (t / 64) % 4, wave = t / 256;
  const int h = 16 * (wave & 3) + (lane & 15);
  const int d0 = 128 * (wave >> 2) + 32 * s + 8 * (lane >> 4);
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = h < a.n_attn_heads ? a.q_attn[sess][h * 512 + d0 + i] : 0.0f;
  v8bf t0, t1, t2;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __bf16 a0, a1, a2;
    split3_bf16(x[i], a0, a1, a2);
    t0[i] = a0;
    t1[i] = a1;
    t2[i] = a2;
  }
  uint4 *dst = a.attn_out + (size_t)sess * kAttnQVecs;
  dst[attn_q_index(wave, s, 0, lane)] = __builtin_bit_cast(uint4, t0);
  dst[attn_q_index(wave, s, 1, lane)] = __builtin_bit_cast(uint4, t1);
  dst[attn_q_index(wave, s, 2, lane)] = __builtin_bit_cast(uint4, t2);
}

__global__ void __launch_bounds__(kSplitThreads) q_split_kernel(const QSplitArgs a) {
  const int sess = blockIdx.y;
  if ((int)blockIdx.x >= a.idx_blocks) {
    attn_q_split(a, sess, (blockIdx.x - a.idx_blocks) * kSplitThreads + threadIdx.x);
    return;
  }
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
                          uint32_t *out, const float *const *q_attn, int n_attn_heads, uint4 *attn_out,
                          hipStream_t st) {
  QSplitArgs a;
  for (int i = 0; i < n_sessions; ++i) {
    a.q[i] = q ? q[i] : nullptr;
    a.w[i] = w ? w[i] : nullptr;
    a.q_attn[i] = q_attn ? q_attn[i] : nullptr;
  }
  a.out = out;
  a.attn_out = attn_out;
  a.n_heads = n_heads;
  a.n_attn_heads = n_attn_heads;
  a.idx_blocks = q ? kSplitBlocks : 0;
  const int blocks = a.idx_blocks + (q_attn ? kAttnSplitBlocks : 0);
  if (blocks == 0) return hipSuccess;
  q_split_kernel<<<dim3(blocks, n_sessions), kSplitThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa
