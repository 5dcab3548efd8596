// csa_internal.hpp -- launchers shared between the library's translation
// units.  Each launcher only enqueues work on `stream`; arguments have been
// validated by the C-ABI layer (csa_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

// Tile of the score kernel: rows scored by one workgroup and kept in LDS.
constexpr int kMaxTileRows = 2048;
constexpr int kMinTileRows = 512;
// Heads per tile: the tile's exact top-H keys, H in {8, 16, 32, 64}.
constexpr int kMinTileHeads = 8;
constexpr int kMaxTileHeads = 64;

// Heads per tile for a session of nt tiles: enough that the heads of all
// tiles number at least ~2048 (so few tiles hold more winners than heads),
// or ~1024 once a tile keeps 32 (the exact top-64 of a tile costs several
// histogram passes, and 1024 heads still bound the 512th key well).  With
// at most 512 heads possible the bound is 1 whatever hd is.
inline int heads_per_tile(int64_t nt) {
  // too few tiles for their heads to bound the 512th key: every tile is
  // read back whole by the selection, so the cheapest heads will do
  if (nt * kMaxTileHeads <= 512) return kMinTileHeads;
  int hd = kMinTileHeads;
  while (hd < kMaxTileHeads && nt * hd < 2048 && !(hd >= 32 && nt * hd >= 1024)) hd *= 2;
  return hd;
}

// One launch of the score kernel (csa_topk_tile.hip).
struct TileJob {
  enum Mode { kFilter, kArray, kBounds } mode;  // score + heads; given scores + heads; score + brackets only
  int n_sessions;
  int n_idx_heads;
  int tile_rows;
  const uint8_t *idx_rows[CSA_MAX_SESSIONS];
  const float *scores_in[CSA_MAX_SESSIONS];  // kArray
  int64_t n_rows[CSA_MAX_SESSIONS];
  int hd[CSA_MAX_SESSIONS];
  const float *q[CSA_MAX_SESSIONS];       // indexer query [n_idx_heads][128] (scoring modes)
  const float *w[CSA_MAX_SESSIONS];       // indexer head weights
  uint64_t *hkey;   // [session][heads_stride]: head keys by upper bound, rank-major [hd][nt]
  uint64_t *hlow;   // [session][heads_stride]: their lower-bound keys, same order
  uint64_t *hnext;  // [session][tiles_stride]: per tile its (hd+1)-th key
  int64_t heads_stride, tiles_stride;
  float *bnd_up, *bnd_lo;  // kBounds: the brackets of every row (one session)
  int query_format;        // kQueryFp32 or kQueryMxfp4 (csa_score.hpp)
  float *qhat;             // kQueryMxfp4: the quantized query of every session, [session][64][128] (or null)
};

// Waves per workgroup of the exact rescoring.
constexpr int kRefineWaves = 8;

// One launch of the exact rescoring (csa_refine.hip).
struct RefineJob {
  // kDecode: the filter's candidates scored exactly; kArray: candidates from
  // given scores; kAll: every row's exact score (csa_score); kKeysAll: every
  // row's exact key as an item (the decode step of short histories)
  enum Mode { kDecode, kArray, kAll, kKeysAll } mode;
  int n_sessions;
  int n_idx_heads;
  int tile_rows;
  int k;
  int blocks;  // workgroups per session
  const uint8_t *idx_rows[CSA_MAX_SESSIONS];
  const float *q[CSA_MAX_SESSIONS];
  const float *w[CSA_MAX_SESSIONS];
  float *scores[CSA_MAX_SESSIONS];  // kArray: the given scores; kAll: the output
  int64_t n_rows[CSA_MAX_SESSIONS];
  int hd[CSA_MAX_SESSIONS];
  const float *q_attn[CSA_MAX_SESSIONS];  // kDecode: the attention query [n_attn_heads][512]
  uint4 *attn_q;                          // kDecode: its split, [session][kAttnQVecs] (null: none)
  int n_attn_heads;
  const uint64_t *hkey;  // rank-major heads (TileJob)
  const uint64_t *hlow;
  const uint64_t *hnext;
  uint64_t *items;  // [session][items_stride]
  uint32_t *count;  // [session]
  int64_t heads_stride, tiles_stride, items_stride;
};

// One launch of the global selection (and, optionally, of the attention
// of the selected rows).
struct SelectJob {
  int n_sessions;
  int k;
  int slices;          // workgroups per session
  bool array_scores;   // sel_score from the score array (csa_topk) or the key
  const float *scores[CSA_MAX_SESSIONS];
  int64_t n_rows[CSA_MAX_SESSIONS];
  int32_t *sel_idx[CSA_MAX_SESSIONS];
  float *sel_score[CSA_MAX_SESSIONS];
  const uint64_t *items;  // [session][items_stride]: exact keys of the rows that can reach the top-k
  const uint32_t *count;  // [session]
  int64_t items_stride;
  // attention partials of the selected rows (attn_part == nullptr: none);
  // then slices must equal kAttnSlices (row groups x head groups)
  const uint4 *attn_q;  // [session][attention query split]
  float *attn_part;     // [session][group][64][512]
  float *attn_ml;       // [session][group][64][2]
  const uint8_t *kv_rows[CSA_MAX_SESSIONS];
  int n_heads;
  float softmax_scale;
};

// Per-session pointers of the attention stages.
struct AttnSession {
  const uint8_t *kv_rows;
  const int32_t *sel_idx;
  const float *q_attn;
  float *out;
  float *lse;
  int64_t n_rows;
  int32_t n_sel;
};


hipError_t launch_dequant_idx(const uint8_t *rows, int64_t n, float *out, hipStream_t st);
hipError_t launch_dequant_kv(const uint8_t *rows, int64_t n, float *out, hipStream_t st);
// MXFP4 quantization of an indexer query [n_heads][128] into rows [n_heads][68].
hipError_t launch_quantize_query(const float *q, int n_heads, uint8_t *rows, hipStream_t st);
// Attention query split of every session (csa_qsplit.hip): q_attn[i] ->
// attn_out + i * kAttnQVecs.
hipError_t launch_attn_q_split(const float *const *q_attn, int n_sessions, int n_attn_heads, uint4 *attn_out,
                               hipStream_t st);
// Dense attention (csa_dense_attn): at most kDenseMaxGroups groups of a
// multiple of 32 rows (at most 512), as few rows per group as that allows.
constexpr int kDenseMaxGroups = 256;
inline void dense_grouping(int64_t n_rows, int *rows_per_group, int *groups) {
  const int64_t per = 32 * ((n_rows + 32 * kDenseMaxGroups - 1) / (32 * kDenseMaxGroups));
  *rows_per_group = (int)(per > 32 ? per : 32);
  *groups = (int)((n_rows + *rows_per_group - 1) / *rows_per_group);
}
// Partials and the merge of a dense attention (csa_attn.hip); qsplit holds
// the attention query split (launch_attn_q_split).
hipError_t launch_dense_attn(const uint8_t *kv_rows, int64_t n_rows, const uint4 *qsplit, int n_heads, float scale,
                             float *part, float *ml, float *out, float *lse, hipStream_t st);
// New rows packed into the 583/68-byte formats (csa_pack.hip); either
// value array may be null.
hipError_t launch_pack(const float *kv_vals, const float *idx_vals, int64_t n, uint8_t *kv_rows, uint8_t *idx_rows,
                       hipStream_t st);
// The merge of two attention results over disjoint rows (csa_pack.hip).
hipError_t launch_lse_merge(const float *out_a, const float *lse_a, const float *out_b, const float *lse_b,
                            int n_heads, float *out, float *lse, hipStream_t st);
// With ev_start and ev_end (both or neither) the scoring launch records them
// at its own start and end (hipExtLaunchKernelGGL), so they time the kernel
// itself rather than the queue around it.
hipError_t launch_tiles(const TileJob &job, hipStream_t st, hipEvent_t ev_start = nullptr,
                        hipEvent_t ev_end = nullptr);
hipError_t launch_refine(const RefineJob &job, hipStream_t st);
hipError_t launch_select(const SelectJob &job, hipStream_t st);
// Attention partials of the rows sel_idx[0..n_sel) of every session, one
// workgroup per group (csa_sparse_attn).
// 2^groups_lg row groups per session (at most 32; the fused selection uses 32).
hipError_t launch_attn_rows(const AttnSession *s, int n_sessions, int n_heads, float softmax_scale,
                            const uint4 *qsplit, float *part, float *ml, int groups_lg, hipStream_t st);
// Merge of the group partials: out, lse.
hipError_t launch_attn_combine(const AttnSession *s, int n_sessions, int n_heads, const float *part,
                               const float *ml, int groups_lg, hipStream_t st);

}  // namespace csa
