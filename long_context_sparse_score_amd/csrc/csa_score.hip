// csa_score.hip -- indexer score of every packed row (csa_score).
//
// Score (the lightning-indexer form adopted for the whole library; the DS4X
// page describes the batch-one scorer only as a block-scaled MXFP4 matrix
// product over the 68-byte rows, "Optimization details"):
//   s_j = sum_h w_h * max(0, q_h . k_j)
// The order of operations is fixed so that a row's fp32 score depends only
// on its bytes: each head's dot product is an FMA chain over i = 0..127
// starting from 0, heads are accumulated with FMAs for h = 0..H-1, and -0 is
// stored as +0.  score_row() is the single definition of that order.
#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "csa_score.hpp"

namespace csa {

struct ScoreArgs {
  ScoreSession s[CSA_MAX_SESSIONS];
  int n_idx_heads;
};

// One thread per row; blockIdx.y selects the session.
__global__ void __launch_bounds__(256) score_rows_kernel(const ScoreArgs a) {
  const ScoreSession &S = a.s[blockIdx.y];
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= S.n_rows) return;
  const uint32_t *w = reinterpret_cast<const uint32_t *>(S.idx_rows + j * kIdxRowBytes);
  uint32_t words[17];
#pragma unroll
  for (int d = 0; d < 17; ++d) words[d] = w[d];
  S.scores[j] = score_row(words, S.q_idx, S.w_idx, a.n_idx_heads);
}

hipError_t launch_score(const ScoreSession *s, int n_sessions, int n_idx_heads, int64_t max_rows,
                        hipStream_t st) {
  if (max_rows == 0) return hipSuccess;
  ScoreArgs a;
  for (int i = 0; i < n_sessions; ++i) a.s[i] = s[i];
  a.n_idx_heads = n_idx_heads;
  dim3 grid((unsigned)((max_rows + 255) / 256), (unsigned)n_sessions);
  score_rows_kernel<<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa
