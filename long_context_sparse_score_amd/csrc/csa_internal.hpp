// csa_internal.hpp -- launchers shared between the library's translation
// units.  Each launcher only enqueues work on `stream`; arguments have been
// validated by the C-ABI layer (csa_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

// Largest tile of the score/select kernel (rows kept in LDS as 32-bit
// order keys) and the smallest (the tile's top-512 needs >= 512 rows).
constexpr int kMaxTileRows = 4096;
constexpr int kMinTileRows = 512;

// One launch of the tile kernel (and of the merge that follows it).
struct TileJob {
  enum Mode { kScore, kScoreSelect, kArraySelect } mode;
  int n_sessions;
  int n_idx_heads;
  int tile_rows;
  const uint8_t *idx_rows[CSA_MAX_SESSIONS];
  const float *scores_in[CSA_MAX_SESSIONS];
  float *scores_out[CSA_MAX_SESSIONS];
  int64_t n_rows[CSA_MAX_SESSIONS];
  const uint32_t *qsplit;  // query split, [session][kQSplitBytes / 4]
  uint64_t *cand;          // per tile: its top-512 keys
  uint64_t *heads;         // per tile: its top-16 keys, sorted
  int64_t cand_stride, heads_stride;  // keys per session
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
// Query split of every session (csa_qsplit.hip): q[i], w[i] -> out.
hipError_t launch_q_split(const float *const *q, const float *const *w, int n_sessions, int n_heads,
                          uint32_t *out, hipStream_t st);
hipError_t launch_tiles(const TileJob &job, hipStream_t st);
hipError_t launch_merge(const TileJob &job, int32_t *const *sel_idx, float *const *sel_score, int k,
                        hipStream_t st);
// part: workspace of n_sessions * kAttnPartFloats floats (session-major).
hipError_t launch_attention(const AttnSession *s, int n_sessions, int n_heads, float softmax_scale,
                            float *part, hipStream_t st);

}  // namespace csa
