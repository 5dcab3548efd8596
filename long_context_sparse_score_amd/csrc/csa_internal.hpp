// csa_internal.hpp -- launchers shared between the library's translation
// units.  Each launcher only enqueues work on `stream`; arguments have been
// validated by the C-ABI layer (csa_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

// Per-session pointers for the indexer-score stage.
struct ScoreSession {
  const uint8_t *idx_rows;
  const float *q_idx;
  const float *w_idx;
  float *scores;
  int64_t n_rows;
};

// Per-session pointers for the selection stage.
struct SelectSession {
  const float *scores;
  int32_t *sel_idx;
  float *sel_score;
  int64_t n_rows;
};

// Per-session pointers for the attention stages.
struct AttnSession {
  const uint8_t *kv_rows;
  const int32_t *sel_idx;
  const float *q_attn;
  float *out;
  float *lse;
  int64_t n_rows;
  int32_t n_sel;
};

// Attention split: rows of the selection handled by one workgroup.
constexpr int kAttnRowsPerSplit = 16;
constexpr int kAttnSplits = CSA_TOPK / kAttnRowsPerSplit;  // 32
constexpr int kAttnHeadsPerGroup = 16;
// Floats of split partials per session: [split][head][512 acc + m + l].
constexpr size_t kAttnPartFloats = (size_t)kAttnSplits * CSA_MAX_HEADS * (CSA_KV_DIM + 2);

hipError_t launch_dequant_idx(const uint8_t *rows, int64_t n, float *out, hipStream_t st);
hipError_t launch_dequant_kv(const uint8_t *rows, int64_t n, float *out, hipStream_t st);
hipError_t launch_score(const ScoreSession *s, int n_sessions, int n_idx_heads, int64_t max_rows,
                        hipStream_t st);
hipError_t launch_select(const SelectSession *s, int n_sessions, int k, hipStream_t st);
// part: workspace of n_sessions * kAttnPartFloats floats (session-major).
hipError_t launch_attention(const AttnSession *s, int n_sessions, int n_heads, float softmax_scale,
                            float *part, hipStream_t st);

}  // namespace csa
