// csa_qsplit.hip -- the attention query split for csa_sparse_attn and
// csa_dense_attn: three bf16 terms per value in the matrix-core operand order
// of csa_attn.hpp (attn_q_split_task).  The decode step does the same split
// inside the exact rescoring kernel (a share per workgroup), and the indexer
// query is split in registers by the score kernel's waves (csa_score.hpp), so
// this launch serves the stand-alone attention only.
#include "csa_attn.hpp"
#include "csa_internal.hpp"

namespace csa {

struct QSplitArgs {
  const float *q_attn[CSA_MAX_SESSIONS];
  uint4 *attn_out;  // [session][kAttnQVecs]
  int n_attn_heads;
};

constexpr int kSplitThreads = 256;

__global__ void __launch_bounds__(kSplitThreads) q_split_kernel(const QSplitArgs a) {
  const int sess = blockIdx.y;
  attn_q_split_task(a.q_attn[sess], a.n_attn_heads, a.attn_out + (size_t)sess * kAttnQVecs,
                    blockIdx.x * kSplitThreads + threadIdx.x);
}

hipError_t launch_attn_q_split(const float *const *q_attn, int n_sessions, int n_attn_heads, uint4 *attn_out,
                               hipStream_t st) {
  QSplitArgs a;
  for (int i = 0; i < n_sessions; ++i) a.q_attn[i] = q_attn[i];
  a.attn_out = attn_out;
  a.n_attn_heads = n_attn_heads;
  q_split_kernel<<<dim3(kAttnQTasks / kSplitThreads, n_sessions), kSplitThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa
