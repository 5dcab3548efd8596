// csa_attn.hip -- softmax attention over selected packed KV rows (DS4X page,
// kernel group "indexed attention"; row layout from "Packed cache ABI"):
//   l[h][j] = scale * q_h . kv_j,   out[h] = sum_j softmax(l[h])_j kv_j,
//   lse[h] = log sum_j exp(l[h][j]),
// split over kAttnGroups groups of rows (csa_attn.hpp) and merged here.
//   attn_rows_kernel  grid (kAttnSlices, sessions): the partial of row group
//                     b % 32 for head group b / 32, over the entries of
//                     sel_idx[0..n_sel) that belong to the row group
//                     (csa_sparse_attn; the decode step computes the same
//                     partials inside its selection kernel);
//   attn_combine      one thread per (head, dimension): merges the groups.
// Entries of sel_idx outside [0, n_rows) contribute nothing; with no valid
// entry out = 0 and lse = -inf.
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
};
static_assert(sizeof(AttnArgs) <= 4096, "kernel argument block");

// ---------------------------------------------------------------- group partials

struct RowsShared {
  AttnStage st;
  int32_t key[CSA_TOPK + 16], row[CSA_TOPK], ordered[CSA_TOPK];
  uint32_t cnt;
};

__global__ void __launch_bounds__(kAttnThreads) attn_rows_kernel(const AttnArgs a) {
  const int sess = blockIdx.y, grp = blockIdx.x % kAttnGroups, hg = blockIdx.x / kAttnGroups;
  const AttnSession &S = a.s[sess];
  __shared__ RowsShared sh;
  if (threadIdx.x == 0) sh.cnt = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < S.n_sel; j += kAttnThreads) {
    const int32_t r = S.sel_idx[j];
    if (r >= 0 && (int64_t)r < S.n_rows && attn_group((uint32_t)r) == (uint32_t)grp) {
      const uint32_t p = atomicAdd(&sh.cnt, 1u);
      sh.key[p] = j;
      sh.row[p] = r;
    }
  }
  __syncthreads();
  const int m = (int)sh.cnt;
  attn_order(sh.key, sh.row, m, sh.ordered);
  attn_group_rows(a.qsplit + (size_t)sess * kAttnQVecs, sh.st, sh.ordered, m, S.kv_rows, a.softmax_scale, a.n_heads, hg,
                  a.part + (size_t)sess * kAttnPartFloats + (size_t)grp * CSA_MAX_HEADS * kKvDim,
                  a.ml + (size_t)sess * kAttnMlFloats + (size_t)grp * CSA_MAX_HEADS * 2);
}

// ---------------------------------------------------------------- combine

constexpr int kCombineThreads = 256;

__global__ void __launch_bounds__(kCombineThreads) attn_combine_kernel(const AttnArgs a) {
  const int sess = blockIdx.y;
  const AttnSession &S = a.s[sess];
  const int e = blockIdx.x * kCombineThreads + threadIdx.x;  // head * 512 + dimension
  const int h = e / kKvDim;
  if (h >= a.n_heads) return;
  float lse;
  S.out[e] = attn_merge_element(a.ml + (size_t)sess * kAttnMlFloats, a.part + (size_t)sess * kAttnPartFloats, h, e, lse);
  if (S.lse && e % kKvDim == 0) S.lse[h] = lse;
}

// ---------------------------------------------------------------- launchers

static AttnArgs attn_args(const AttnSession *s, int n_sessions, int n_heads, float scale, const uint4 *qsplit,
                          float *part, float *ml) {
  AttnArgs a;
  for (int i = 0; i < n_sessions; ++i) a.s[i] = s[i];
  a.qsplit = qsplit;
  a.part = part;
  a.ml = ml;
  a.n_heads = n_heads;
  a.softmax_scale = scale;
  return a;
}

hipError_t launch_attn_rows(const AttnSession *s, int n_sessions, int n_heads, float softmax_scale,
                            const uint4 *qsplit, float *part, float *ml, hipStream_t st) {
  const AttnArgs a = attn_args(s, n_sessions, n_heads, softmax_scale, qsplit, part, ml);
  attn_rows_kernel<<<dim3(kAttnSlices, n_sessions), kAttnThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnSession *s, int n_sessions, int n_heads, const float *part,
                               const float *ml, hipStream_t st) {
  const AttnArgs a =
      attn_args(s, n_sessions, n_heads, 0.0f, nullptr, const_cast<float *>(part), const_cast<float *>(ml));
  const unsigned blocks = (unsigned)((n_heads * kKvDim + kCombineThreads - 1) / kCombineThreads);
  attn_combine_kernel<<<dim3(blocks, n_sessions), kCombineThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa
