// csa_attn.hip -- softmax attention over selected packed KV rows (DS4X page,
// kernel group "indexed attention"; row layout from "Packed cache ABI"):
//   l[h][j] = scale * q_h . kv_j,   out[h] = sum_j softmax(l[h])_j kv_j,
//   lse[h] = log sum_j exp(l[h][j]),
// split over kAttnGroups groups of rows (csa_attn.hpp) and merged here.
//   attn_rows_kernel  grid (4 G, sessions), G = 2^groups_lg row groups: the
//                     partial of row group b % G for head group b / G, over
//                     the entries of sel_idx[0..n_sel) that belong to the
//                     row group
//                     (csa_sparse_attn; the decode step computes the same
//                     partials inside its selection kernel);
//   attn_combine      one thread per (head, dimension): merges the groups.
// Entries of sel_idx outside [0, n_rows) contribute nothing; with no valid
// entry out = 0 and lse = -inf.
// Dense attention (csa_dense_attn; DS4X page, "What DS4X changes" and
// "Optimization details": the HCA layers' exact score-split attention over
// every compressed row, without a row ceiling) splits the rows into up to
// kDenseMaxGroups contiguous groups of a multiple of 32 rows:
//   dense_rows_kernel   grid (4 G): the partial of group b % G for head
//                       group b / G (the same per-group attention);
//   dense_combine       one thread per (head, dimension): merges the G
//                       groups in group order.
#include "csa_attn.hpp"
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

struct AttnArgs {
  AttnSession s[CSA_MAX_SESSIONS];
  const uint4 *qsplit;  // [session][kAttnQVecs]
  float *part;          // [session][kAttnPartFloats]
  float *ml;            // [session][kAttnMlFloats]
  int n_heads;
  float softmax_scale;
  int groups_lg;  // 2^groups_lg row groups per session
};
static_assert(sizeof(AttnArgs) <= 4096, "kernel argument block");

// ---------------------------------------------------------------- group partials

struct RowsShared {
  AttnStage st;
  int32_t ordered[CSA_TOPK];
  uint32_t wcnt[kAttnWaves];
};

// (at least four waves per SIMD: two workgroups share a compute unit)
__global__ void __launch_bounds__(kAttnThreads, 4) attn_rows_kernel(const AttnArgs a) {
  const int groups = 1 << a.groups_lg;
  const int sess = blockIdx.y, grp = blockIdx.x % groups, hg = blockIdx.x / groups;
  const AttnSession &S = a.s[sess];
  __shared__ RowsShared sh;
  // the row group's entries of sel_idx in position order: entry j goes to
  // the number of the group's entries before it (n_sel <= 512 = one pass)
  static_assert(kAttnThreads >= CSA_TOPK, "one entry per thread");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = tid;
  const int32_t r = j < S.n_sel ? S.sel_idx[j] : -1;
  const bool mine = r >= 0 && (int64_t)r < S.n_rows && attn_group((uint32_t)r, a.groups_lg) == (uint32_t)grp;
  const uint64_t bal = __ballot(mine);
  if (lane == 0) sh.wcnt[wave] = (uint32_t)__popcll(bal);
  __syncthreads();
  uint32_t before = 0, m = 0;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) {
    before += w < wave ? sh.wcnt[w] : 0u;
    m += sh.wcnt[w];
  }
  if (mine) sh.ordered[before + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] = r;
  __syncthreads();
  attn_group_rows(a.qsplit + (size_t)sess * kAttnQVecs, sh.st, sh.ordered, (int)m, S.kv_rows, a.softmax_scale, a.n_heads, hg,
                  a.part + (size_t)sess * kAttnPartFloats + (size_t)grp * CSA_MAX_HEADS * kKvDim,
                  a.ml + (size_t)sess * kAttnMlFloats + (size_t)grp * CSA_MAX_HEADS * 2);
}

// ---------------------------------------------------------------- combine

constexpr int kCombineThreads = 64;  // an eighth of the dimensions per workgroup
constexpr int kCombineSplit = kKvDim / kCombineThreads;

// Eight one-wave workgroups per (head, session), one thread per dimension
// (attn_combine_head).
__global__ void __launch_bounds__(kCombineThreads) attn_combine_kernel(const AttnArgs a) {
  const int sess = blockIdx.y, h = blockIdx.x / kCombineSplit;
  const int d0 = (blockIdx.x % kCombineSplit) * kCombineThreads;
  const AttnSession &S = a.s[sess];
  __shared__ CombineShared cs;
  attn_combine_head(a.ml + (size_t)sess * kAttnMlFloats, a.part + (size_t)sess * kAttnPartFloats, 1 << a.groups_lg, h, d0,
                    kCombineThreads, cs, S.out + (size_t)h * kKvDim, S.lse ? S.lse + h : nullptr);
}

// ---------------------------------------------------------------- dense attention

struct DenseArgs {
  const uint8_t *kv_rows;
  int64_t n_rows;
  int rows_per_group;  // a multiple of 32, at most CSA_TOPK
  int groups;          // ceil(n_rows / rows_per_group) <= kDenseMaxGroups
  const uint4 *qsplit;
  float *part;  // [group][64][512]
  float *ml;    // [group][64][2]
  float *out;
  float *lse;
  int n_heads;
  float softmax_scale;
};

__global__ void __launch_bounds__(kAttnThreads, 4) dense_rows_kernel(const DenseArgs a) {
  const int grp = blockIdx.x % a.groups, hg = blockIdx.x / a.groups;
  __shared__ RowsShared sh;
  const int64_t r0 = (int64_t)grp * a.rows_per_group;
  const int64_t left = a.n_rows - r0;  // >= 1: every group holds a row
  const int m = (int)(left < a.rows_per_group ? left : a.rows_per_group);
  for (int i = threadIdx.x; i < m; i += kAttnThreads) sh.ordered[i] = (int32_t)(r0 + i);
  __syncthreads();
  attn_group_rows(a.qsplit, sh.st, sh.ordered, m, a.kv_rows, a.softmax_scale, a.n_heads, hg,
                  a.part + (size_t)grp * CSA_MAX_HEADS * kKvDim, a.ml + (size_t)grp * CSA_MAX_HEADS * 2);
}

// The merge of head h's group partials for dimensions d0 .. d0 + 63 (one
// per thread): M = max_b m_b, w_b = e^{m_b - M}, L = sum_b w_b l_b in group
// order, out[d] = (sum_b w_b acc_b[d]) / L in group order, lse = M + log L
// (out = 0 and lse = -inf without any group).
__global__ void __launch_bounds__(kCombineThreads) dense_combine_kernel(const DenseArgs a) {
  const int h = blockIdx.x / kCombineSplit, t = threadIdx.x;
  const int d = (blockIdx.x % kCombineSplit) * kCombineThreads + t;
  const int G = a.groups;
  __shared__ float wgt[kDenseMaxGroups];
  __shared__ float Ls, lses;
  float M = -__builtin_inff();
  for (int b = t; b < G; b += kCombineThreads) M = fmaxf(M, a.ml[((size_t)b * CSA_MAX_HEADS + h) * 2]);
#pragma unroll
  for (int o = 1; o < kCombineThreads; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, kCombineThreads));
  for (int b = t; b < G; b += kCombineThreads) {
    const float mb = a.ml[((size_t)b * CSA_MAX_HEADS + h) * 2];
    wgt[b] = mb == -__builtin_inff() ? 0.0f : __expf(mb - M);
  }
  __syncthreads();
  if (t == 0) {
    float L = 0.0f;
    for (int b = 0; b < G; ++b) L += wgt[b] * a.ml[((size_t)b * CSA_MAX_HEADS + h) * 2 + 1];
    Ls = L;
    lses = L > 0.0f ? M + logf(L) : -__builtin_inff();
  }
  __syncthreads();
  float X = 0.0f;
  for (int b = 0; b < G; ++b) {
    const float w = wgt[b];
    const float x = a.part[((size_t)b * CSA_MAX_HEADS + h) * kKvDim + d];
    X += w == 0.0f ? 0.0f : w * x;
  }
  const float L = Ls;
  a.out[(size_t)h * kKvDim + d] = L > 0.0f ? X / L : 0.0f;
  if (a.lse && d == 0) a.lse[h] = lses;
}

hipError_t launch_dense_attn(const uint8_t *kv_rows, int64_t n_rows, const uint4 *qsplit, int n_heads, float scale,
                             float *part, float *ml, float *out, float *lse, hipStream_t st) {
  DenseArgs a;
  a.kv_rows = kv_rows;
  a.n_rows = n_rows;
  dense_grouping(n_rows, &a.rows_per_group, &a.groups);
  a.qsplit = qsplit;
  a.part = part;
  a.ml = ml;
  a.out = out;
  a.lse = lse;
  a.n_heads = n_heads;
  a.softmax_scale = scale;
  if (a.groups > 0) dense_rows_kernel<<<dim3((unsigned)(a.groups * kAttnHeadGroups)), kAttnThreads, 0, st>>>(a);
  dense_combine_kernel<<<dim3((unsigned)(n_heads * kCombineSplit)), kCombineThreads, 0, st>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers

static AttnArgs attn_args(const AttnSession *s, int n_sessions, int n_heads, float scale, const uint4 *qsplit,
                          float *part, float *ml, int groups_lg) {
  AttnArgs a;
  a.groups_lg = groups_lg;
  for (int i = 0; i < n_sessions; ++i) a.s[i] = s[i];
  a.qsplit = qsplit;
  a.part = part;
  a.ml = ml;
  a.n_heads = n_heads;
  a.softmax_scale = scale;
  return a;
}

hipError_t launch_attn_rows(const AttnSession *s, int n_sessions, int n_heads, float softmax_scale,
                            const uint4 *qsplit, float *part, float *ml, int groups_lg, hipStream_t st) {
  const AttnArgs a = attn_args(s, n_sessions, n_heads, softmax_scale, qsplit, part, ml, groups_lg);
  attn_rows_kernel<<<dim3((1u << groups_lg) * kAttnHeadGroups, n_sessions), kAttnThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnSession *s, int n_sessions, int n_heads, const float *part,
                               const float *ml, int groups_lg, hipStream_t st) {
  const AttnArgs a = attn_args(s, n_sessions, n_heads, 0.0f, nullptr, const_cast<float *>(part),
                               const_cast<float *>(ml), groups_lg);
  attn_combine_kernel<<<dim3((unsigned)(n_heads * kCombineSplit), n_sessions), kCombineThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa
