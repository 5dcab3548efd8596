// csa_score.hpp -- the per-row indexer score, the one definition used by the
// unfused score kernel and the fused score/select kernel, so both produce
// bit-identical scores.
#pragma once

#include "csa_device.hpp"

namespace csa {

// words[0..15]: the row's 64 E2M1 code bytes, little-endian (element 8d+t in
// bits 4t..4t+3 of word d); words[16]: the four UE8M0 scale bytes.
// q: [H][128] fp32 (wave-uniform address), wt: [H].
__device__ __forceinline__ float score_row(const uint32_t (&words)[17], const float *__restrict__ q,
                                           const float *__restrict__ wt, int H) {
  float k[128];
  const uint32_t sc = words[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    const float scale = ue8m0_scale((sc >> (8 * (d >> 2))) & 255u);
#pragma unroll
    for (int t = 0; t < 8; ++t) k[8 * d + t] = e2m1_value((words[d] >> (4 * t)) & 15u) * scale;
  }
  float s = 0.0f;
  for (int h = 0; h < H; ++h) {
    const float *qh = q + h * 128;
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < 128; ++i) dot = __builtin_fmaf(qh[i], k[i], dot);
    const float relu = dot > 0.0f ? dot : 0.0f;
    s = __builtin_fmaf(wt[h], relu, s);
  }
  return s == 0.0f ? 0.0f : s;
}

}  // namespace csa
