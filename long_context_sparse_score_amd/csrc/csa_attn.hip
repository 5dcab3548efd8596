// csa_attn.hip -- softmax attention over the selected packed KV rows
// (csa_sparse_attn; the DS4X page's "indexed attention" kernel group).
//
// Split-K over the selection: workgroup (split, head group, session) decodes
// its 16 selected rows into LDS (the decoded rows never reach HBM), computes
// the 16 heads x 16 rows logits, the per-head running max m and sum l of
// exp(logit - m), and the partial sums acc[h][:] = sum_t exp(l_t - m) kv_t.
// A second kernel rescales the partials by exp(m_s - M) and divides, the
// usual log-sum-exp recombination.  The decoded row is both key and value.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

struct AttnPartSession {
  const uint8_t *kv_rows;
  const int32_t *sel_idx;
  const float *q_attn;
  int64_t n_rows;
  int32_t n_sel;
};

struct AttnPartArgs {
  AttnPartSession s[CSA_MAX_SESSIONS];
  float *part;  // [session][split][head][514]
  int n_heads;
  float scale;
};

struct AttnCombSession {
  float *out;
  float *lse;
  int32_t n_sel;
};

struct AttnCombArgs {
  AttnCombSession s[CSA_MAX_SESSIONS];
  const float *part;
  int n_heads;
};

static_assert(sizeof(AttnPartArgs) <= 4096, "kernel argument block");
static_assert(sizeof(AttnCombArgs) <= 4096, "kernel argument block");

constexpr int kR = kAttnRowsPerSplit;    // 16 rows per split
constexpr int kHG = kAttnHeadsPerGroup;  // 16 heads per group
constexpr int kPartStride = CSA_KV_DIM + 2;
constexpr int kLdsStride = CSA_KV_DIM + 4;  // rows 4 banks apart

__device__ __forceinline__ float decode_kv_elem(const uint8_t *r, int i) {
  if (i < kKvNope) return e4m3_value(r[i]) * ue8m0_scale(r[576 + (i >> 6)]);
  const int o = kKvNope + 2 * (i - kKvNope);
  return f16_value((uint32_t)r[o] | ((uint32_t)r[o + 1] << 8));
}

__global__ void __launch_bounds__(256) attn_partial_kernel(const AttnPartArgs a) {
  const int split = blockIdx.x, hg = blockIdx.y, sess = blockIdx.z;
  const AttnPartSession &S = a.s[sess];
  const int tid = threadIdx.x;
  __shared__ float kv[kR][kLdsStride];
  __shared__ float prob[kHG][kR];
  __shared__ int64_t rowid[kR];

  const int r0 = split * kR;
  int nr = S.n_sel - r0;
  nr = nr < 0 ? 0 : (nr > kR ? kR : nr);
  if (tid < kR) {
    int64_t idx = -1;
    if (tid < nr) {
      const int32_t v = S.sel_idx[r0 + tid];
      if (v >= 0 && (int64_t)v < S.n_rows) idx = v;
    }
    rowid[tid] = idx;
  }
  __syncthreads();
  // thread -> elements tid and tid + 256 of all 16 rows; every byte load is
  // issued before any is used.  Invalid rows load nothing (the history may
  // be empty, with no row to read) and decode to zero.
  {
    uint32_t lo[kR][2], hi[kR][2], sc[kR][2];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int64_t idx = rowid[r];  // workgroup-uniform
      if (idx < 0) {
        lo[r][0] = lo[r][1] = hi[r][0] = hi[r][1] = sc[r][0] = sc[r][1] = 0;
        continue;
      }
      const uint8_t *row = S.kv_rows + idx * kKvRowBytes;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int i = tid + 256 * hh;
        if (i < kKvNope) {
          lo[r][hh] = row[i];
          sc[r][hh] = row[576 + (i >> 6)];
          hi[r][hh] = 0;
        } else {
          const int o = kKvNope + 2 * (i - kKvNope);
          lo[r][hh] = row[o];
          hi[r][hh] = row[o + 1];
          sc[r][hh] = 0;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kR; ++r) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int i = tid + 256 * hh;
        const float v = (i < kKvNope) ? e4m3_value(lo[r][hh]) * ue8m0_scale(sc[r][hh])
                                      : f16_value(lo[r][hh] | (hi[r][hh] << 8));
        kv[r][i] = rowid[r] >= 0 ? v : 0.0f;
      }
    }
  }
  __syncthreads();

  // logits: thread -> (head h, row r)
  const int h = tid / kR, r = tid % kR;
  const int hglob = hg * kHG + h;
  float logit = -__builtin_inff();
  if (hglob < a.n_heads && rowid[r] >= 0) {
    const float4 *q4 = reinterpret_cast<const float4 *>(S.q_attn + (size_t)hglob * CSA_KV_DIM);
    const float4 *k4 = reinterpret_cast<const float4 *>(&kv[r][0]);
    float dot = 0.0f;
    for (int i = 0; i < CSA_KV_DIM / 4; ++i) {
      const float4 qv = q4[i], kk = k4[i];
      dot = __builtin_fmaf(qv.x, kk.x, dot);
      dot = __builtin_fmaf(qv.y, kk.y, dot);
      dot = __builtin_fmaf(qv.z, kk.z, dot);
      dot = __builtin_fmaf(qv.w, kk.w, dot);
    }
    logit = a.scale * dot;
  }
  float m = logit;
#pragma unroll
  for (int off = kR / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kR));
  const float p = (m == -__builtin_inff()) ? 0.0f : __expf(logit - m);
  float l = p;
#pragma unroll
  for (int off = kR / 2; off > 0; off >>= 1) l += __shfl_xor(l, off, kR);
  prob[h][r] = p;
  float *part = a.part + ((size_t)(sess * kAttnSplits + split) * CSA_MAX_HEADS) * kPartStride;
  if (r == 0 && hglob < a.n_heads) {
    part[(size_t)hglob * kPartStride + CSA_KV_DIM] = m;
    part[(size_t)hglob * kPartStride + CSA_KV_DIM + 1] = l;
  }
  __syncthreads();

  // partial P.V: thread -> dims tid and tid + 256, all heads of the group
  for (int hh = 0; hh < kHG; ++hh) {
    const int hgl = hg * kHG + hh;
    if (hgl >= a.n_heads) break;
    float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int rr = 0; rr < kR; ++rr) {
      const float pr = prob[hh][rr];
      acc0 = __builtin_fmaf(pr, kv[rr][tid], acc0);
      acc1 = __builtin_fmaf(pr, kv[rr][tid + 256], acc1);
    }
    part[(size_t)hgl * kPartStride + tid] = acc0;
    part[(size_t)hgl * kPartStride + tid + 256] = acc1;
  }
}

__global__ void __launch_bounds__(256) attn_combine_kernel(const AttnCombArgs a) {
  const int h = blockIdx.x, sess = blockIdx.y, tid = threadIdx.x;
  const AttnCombSession &S = a.s[sess];
  const int nsplit = (S.n_sel + kR - 1) / kR;
  const float *base = a.part + (size_t)sess * kAttnSplits * CSA_MAX_HEADS * kPartStride + (size_t)h * kPartStride;
  const size_t sstride = (size_t)CSA_MAX_HEADS * kPartStride;
  // every partial load is issued up front (fixed trip counts, clamped)
  float ms[kAttnSplits], ls[kAttnSplits], a0[kAttnSplits], a1[kAttnSplits];
#pragma unroll
  for (int s = 0; s < kAttnSplits; ++s) {
    const float *ps = base + (s < nsplit ? s : 0) * sstride;
    ms[s] = ps[CSA_KV_DIM];
    ls[s] = ps[CSA_KV_DIM + 1];
    a0[s] = ps[tid];
    a1[s] = ps[tid + 256];
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < kAttnSplits; ++s) M = (s < nsplit) ? fmaxf(M, ms[s]) : M;
  float *out = S.out + (size_t)h * CSA_KV_DIM;
  if (M == -__builtin_inff()) {
    out[tid] = 0.0f;
    out[tid + 256] = 0.0f;
    if (tid == 0 && S.lse) S.lse[h] = -__builtin_inff();
    return;
  }
  float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
  for (int s = 0; s < kAttnSplits; ++s) {
    if (s < nsplit && ms[s] != -__builtin_inff()) {
      const float wgt = __expf(ms[s] - M);
      L = __builtin_fmaf(wgt, ls[s], L);
      o0 = __builtin_fmaf(wgt, a0[s], o0);
      o1 = __builtin_fmaf(wgt, a1[s], o1);
    }
  }
  const float inv = 1.0f / L;
  out[tid] = o0 * inv;
  out[tid + 256] = o1 * inv;
  if (tid == 0 && S.lse) S.lse[h] = M + __logf(L);
}

hipError_t launch_attention(const AttnSession *s, int n_sessions, int n_heads, float softmax_scale,
                            float *part, hipStream_t st) {
  AttnPartArgs pa;
  AttnCombArgs ca;
  for (int i = 0; i < n_sessions; ++i) {
    pa.s[i] = AttnPartSession{s[i].kv_rows, s[i].sel_idx, s[i].q_attn, s[i].n_rows, s[i].n_sel};
    ca.s[i] = AttnCombSession{s[i].out, s[i].lse, s[i].n_sel};
  }
  pa.part = part;
  ca.part = part;
  pa.n_heads = n_heads;
  ca.n_heads = n_heads;
  pa.scale = softmax_scale;
  dim3 g1(kAttnSplits, (n_heads + kHG - 1) / kHG, n_sessions);
  attn_partial_kernel<<<g1, 256, 0, st>>>(pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(n_heads, n_sessions);
  attn_combine_kernel<<<g2, 256, 0, st>>>(ca);
  return hipGetLastError();
}

}  // namespace csa
