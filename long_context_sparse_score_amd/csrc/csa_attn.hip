// csa_attn.hip -- softmax attention over the selected packed KV rows (DS4X
// page, kernel group "indexed attention"; row layout from "Packed cache
// ABI"): the decoded 512-value row is both key and value,
//   l[h][j] = scale * q_h . kv_j,   out[h] = sum_j softmax(l[h])_j kv_j,
//   lse[h] = log sum_j exp(l[h][j]).
// Two kernels:
//   logits_kernel  the logits of rows sel_idx[0..n_sel) (csa_attn.hpp), for
//                  csa_sparse_attn; the decode step computes the same values
//                  inside its selection kernel;
//   pv_kernel      grid (32 dimension tiles of 16, sessions), 4 waves = 4
//                  head groups: the softmax of each head over its logits,
//                  then out = P V on the bf16 matrix cores, with P = hi + lo
//                  (two bf16 terms, residual below 2^-17 of each weight) and
//                  V exact (one bf16 term, two for the FP16 RoPE values).
// Entries of sel_idx outside [0, n_rows) contribute nothing; with no valid
// entry out = 0 and lse = -inf.
#include "csa_attn.hpp"
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

struct AttnArgs {
  AttnSession s[CSA_MAX_SESSIONS];
  float *logits;  // [session][64][512]
  int n_heads;
  float softmax_scale;
};
static_assert(sizeof(AttnArgs) <= 4096, "kernel argument block");

__device__ __forceinline__ bool valid_row(int32_t r, int64_t n) { return r >= 0 && (int64_t)r < n; }

// ---------------------------------------------------------------- logits

constexpr int kLogitBatches = CSA_TOPK / kLogitRows;  // 32

__global__ void __launch_bounds__(kLogitThreads) logits_kernel(const AttnArgs a) {
  const int sess = blockIdx.y;
  const AttnSession &S = a.s[sess];
  const int p0 = blockIdx.x * kLogitRows;
  if (p0 >= S.n_sel) return;
  const int nb = S.n_sel - p0 < kLogitRows ? S.n_sel - p0 : kLogitRows;
  __shared__ LogitShared sh;
  LogitQueryRaw qraw;
  load_logit_query(qraw, S.q_attn, a.n_heads);
  const int tid = threadIdx.x;
  if (tid < kLogitRows) {
    const int32_t r = tid < nb ? S.sel_idx[p0 + tid] : -1;
    sh.row[tid] = valid_row(r, S.n_rows) ? r : -1;
    sh.pos[tid] = p0 + tid;
  }
  __syncthreads();
  decode_logit_rows(S.kv_rows, S.n_rows > 0, sh, nb);
  LogitQuery q;
  split_logit_query(q, qraw);
  __syncthreads();
  batch_logits(q, sh, nb, a.n_heads, a.softmax_scale, a.logits + (size_t)sess * kLogitFloats);
}

// ---------------------------------------------------------------- softmax + PV

constexpr int kPvThreads = 256;
constexpr int kPvTileDims = 16;
constexpr int kPvTiles = kKvDim / kPvTileDims;  // 32
constexpr int kPvStride = kPvTileDims + 1;

struct PvShared {
  float v[CSA_TOPK][kPvStride];  // value tile: selected row x 16 dimensions
  int32_t row[CSA_TOPK];
};

__global__ void __launch_bounds__(kPvThreads) pv_kernel(const AttnArgs a) {
  const int sess = blockIdx.y;
  const AttnSession &S = a.s[sess];
  const int dt = blockIdx.x;
  const int tid = threadIdx.x, g = tid >> 6, lane = tid & 63;
  const int n_sel = S.n_sel;
  __shared__ PvShared sh;
  for (int j = tid; j < CSA_TOPK; j += kPvThreads) {
    const int32_t r = j < n_sel ? S.sel_idx[j] : -1;
    sh.row[j] = valid_row(r, S.n_rows) ? r : -1;
  }
  // this lane's logits: head 16g + l%16, rows 32 s + 8 (l/16) + i
  const int h = 16 * g + (lane & 15);
  const bool head_ok = h < a.n_heads;
  const float *lg = a.logits + (size_t)sess * kLogitFloats + (size_t)(head_ok ? h : 0) * CSA_TOPK;
  // every slot of the logits buffer is readable: load all 512 without
  // conditions (a condition would let the compiler put each load behind its
  // own branch and wait), mask after the barrier
  float p[16][8];
#pragma unroll
  for (int s = 0; s < 16; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) p[s][i] = lg[32 * s + 8 * (lane >> 4) + i];
  __syncthreads();
  // value tile: 512 rows x 16 dimensions, 32 per thread
  const int d0 = kPvTileDims * dt;
  if (S.n_rows > 0) {
    constexpr int U = CSA_TOPK * kPvTileDims / kPvThreads;
    int32_t r[U];
    uint32_t b0[U], b1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = sh.row[(tid + kPvThreads * u) / kPvTileDims];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = tid + kPvThreads * u;
      kv_load(S.kv_rows + (size_t)(uint32_t)max(r[u], 0) * kKvRowBytes, d0 + e % kPvTileDims, b0[u], b1[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = tid + kPvThreads * u;
      const float x = kv_decode(d0 + e % kPvTileDims, b0[u], b1[u]);
      sh.v[e / kPvTileDims][e % kPvTileDims] = r[u] >= 0 ? x : 0.0f;
    }
  } else {
    for (int e = tid; e < CSA_TOPK * kPvTileDims; e += kPvThreads) sh.v[e / kPvTileDims][e % kPvTileDims] = 0.0f;
  }
  // invalid entries (and entries past n_sel, and absent heads) carry no weight
#pragma unroll
  for (int s = 0; s < 16; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i)
    {
      const bool bad = (sh.row[32 * s + 8 * (lane >> 4) + i] < 0) | !head_ok;
      p[s][i] = bad ? -__builtin_inff() : p[s][i];
    }
  float m = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < 16; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, p[s][i]);
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  const float mref = m == -__builtin_inff() ? 0.0f : m;
  float sum = 0.0f;
#pragma unroll
  for (int s = 0; s < 16; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[s][i] = __expf(p[s][i] - mref);
      sum += p[s][i];
    }
  sum += __shfl_xor(sum, 16, 64);
  sum += __shfl_xor(sum, 32, 64);
  __syncthreads();  // value tile complete
  const bool rope = d0 >= kKvNope;
  v4f_attn c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    v8bf ph, pl, vh, vl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ph[i] = (__bf16)p[s][i];
      pl[i] = (__bf16)(p[s][i] - (float)ph[i]);
      const float v = sh.v[32 * s + 8 * (lane >> 4) + i][lane & 15];
      vh[i] = (__bf16)v;
      vl[i] = (__bf16)(v - (float)vh[i]);
    }
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vh, c, 0, 0, 0);
    if (rope) {
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vl, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vl, c, 0, 0, 0);
    }
  }
  // lane l holds heads 16g + 4(l/16) + v, dimension d0 + l%16; the sum and
  // maximum of head 16g + x sit in lane x
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int src = 4 * (lane >> 4) + v;
    const float sv = __shfl(sum, src, 64);
    const int hv = 16 * g + src;
    if (hv < a.n_heads) S.out[(size_t)hv * kKvDim + d0 + (lane & 15)] = sv > 0.0f ? c[v] / sv : 0.0f;
  }
  if (dt == 0 && lane < 16 && head_ok && S.lse) S.lse[h] = sum > 0.0f ? mref + logf(sum) : -__builtin_inff();
}

// ---------------------------------------------------------------- launchers

static AttnArgs attn_args(const AttnSession *s, int n_sessions, int n_heads, float scale, const float *logits) {
  AttnArgs a;
  for (int i = 0; i < n_sessions; ++i) a.s[i] = s[i];
  a.logits = const_cast<float *>(logits);
  a.n_heads = n_heads;
  a.softmax_scale = scale;
  return a;
}

hipError_t launch_logits(const AttnSession *s, int n_sessions, int n_heads, float softmax_scale, float *logits,
                         hipStream_t st) {
  const AttnArgs a = attn_args(s, n_sessions, n_heads, softmax_scale, logits);
  logits_kernel<<<dim3(kLogitBatches, n_sessions), kLogitThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_pv(const AttnSession *s, int n_sessions, int n_heads, const float *logits, hipStream_t st) {
  const AttnArgs a = attn_args(s, n_sessions, n_heads, 0.0f, logits);
  pv_kernel<<<dim3(kPvTiles, n_sessions), kPvThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa
