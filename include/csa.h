/*
 * csa.h -- C ABI of the MI355X (gfx950) CSA decode-step library, libcsa.so.
 *
 * The operation: one decode step of DeepSeek-V4-Flash compressed sparse
 * attention (CSA) over a packed, compressed KV history, as described on the
 * DS4X page: the batch-one indexer scores the query against every packed
 * 68-byte indexer row ("Optimization details"), the exact top-512 rows are
 * selected with float score order and lower-index tie break ("CSA
 * score/top-512 fusion"), and attention runs over only those packed 583-byte
 * KV rows ("Packed cache ABI"; kernel group "indexed attention" in the 1M
 * Nsight table).
 *
 * Conventions shared by every entry point
 *  - Pointers named *_rows, q_*, w_*, scores, sel_*, out, lse and ws are
 *    DEVICE pointers owned by the caller.  The library allocates no device
 *    memory; scratch space comes from the caller's workspace `ws`, which must
 *    be 256-byte aligned and at least csa_workspace_bytes(...) long.  Only
 *    the csa_session array passed to csa_decode_step lives in HOST memory and
 *    is read before the call returns.
 *  - `hip_stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work on it and returns; results are valid once
 *    the stream reaches that point.  Calls on one workspace must not overlap.
 *  - Return value: CSA_OK, or a negative csa_status.  Arguments are checked
 *    on the host before anything is launched; on an error nothing is
 *    enqueued and outputs are untouched.  CSA_EDEVICE reports a HIP error at
 *    launch time; CSA_EUNSUPPORTED a device that is not gfx950.
 *  - Data validity is not checked on the device: NaN scale bytes (0xFF) or
 *    NaN E4M3 codes give deterministic results outside the accuracy contract.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 2u

/* Indexer row (DS4X page, "Packed cache ABI"): 128 E2M1 codes, two per byte,
 * element 2i in the low nibble (64 B), then 4 UE8M0 scales, scale b covering
 * elements [32b, 32b+32).  68 bytes, rows densely packed. */
#define CSA_IDX_ROW_BYTES 68
#define CSA_IDX_DIM 128
/* KV row (same section): 448 E4M3 (OCP "FN") non-RoPE bytes, 64 little-endian
 * FP16 RoPE values (128 B), 7 UE8M0 scales, scale b covering non-RoPE
 * elements [64b, 64b+64); the RoPE tail is unscaled.  583 bytes, 512
 * elements, rows densely packed (no alignment). */
#define CSA_KV_ROW_BYTES 583
#define CSA_KV_DIM 512
#define CSA_KV_NOPE 448
/* Indexer query formats of the decode step.  CSA_QUERY_FP32 scores the fp32
 * query as given.  CSA_QUERY_MXFP4 scores the query quantized to MXFP4
 * (csa_quantize_query), the block-scaled MXFP4 scorer of the DS4X page ("What
 * DS4X changes", "Optimization details"): every score is then that of the
 * decoded quantized query, computed exactly as csa_score does. */
#define CSA_QUERY_FP32 0
#define CSA_QUERY_MXFP4 1
/* Rows kept by the selection. */
#define CSA_TOPK 512
/* Limits checked by every entry point. */
#define CSA_MAX_HEADS 64
#define CSA_MAX_SESSIONS 64
#define CSA_MAX_ROWS (((int64_t)1) << 30)

typedef enum csa_status {
  CSA_OK = 0,
  CSA_EINVAL = -1,       /* a null pointer, a size out of range, a misaligned row buffer */
  CSA_EWORKSPACE = -2,   /* workspace too small or not 256-byte aligned */
  CSA_EDEVICE = -3,      /* a HIP runtime error while enqueueing */
  CSA_EUNSUPPORTED = -4  /* the current device is not gfx950 */
} csa_status;

/* One decode session: its own history and its own query token. */
typedef struct csa_session {
  const uint8_t *idx_rows; /* [n_rows][68] indexer rows, 16-byte aligned */
  const uint8_t *kv_rows;  /* [n_rows][583] KV rows */
  int64_t n_rows;          /* 0 <= n_rows <= CSA_MAX_ROWS */
  const float *q_idx;      /* [n_idx_heads][128] indexer query, 16-byte aligned */
  const float *w_idx;      /* [n_idx_heads] per-head indexer weights */
  const float *q_attn;     /* [n_heads][512] attention query */
  int32_t *sel_idx;        /* out [512]: selected rows, best first, -1 padded */
  float *sel_score;        /* out [512] or NULL: their scores, -inf padded */
  float *out;              /* out [n_heads][512] attention output */
  float *lse;              /* out [n_heads] or NULL: natural-log sum-exp */
} csa_session;

/* CSA_ABI_VERSION of the loaded library. */
uint32_t csa_abi_version(void);

/* Static text for a csa_status value. */
const char *csa_strerror(int status);

/* Workspace bytes every entry point needs for sessions of up to
 * `max_rows_per_session` rows (0 if the arguments are out of range).  The
 * same workspace serves csa_score, csa_topk, csa_sparse_attn and
 * csa_decode_step; its contents need no initialisation and are scratch
 * between calls. */
size_t csa_workspace_bytes(int64_t max_rows_per_session, int n_sessions);

/* Indexer score of every row (the legacy first stage; DS4X page, "What DS4X
 * changes": full F32 score array, then a separate exact top-512 pass):
 *   scores[j] = sum_h w_idx[h] * max(0, sum_i q_idx[h][i] * k_j[i]),
 * k_j the decoded row j (each value an E2M1 code times its block's
 * 2^(e-127), as fp32).  Computed in fp64 with i ascending inside a head and h
 * ascending outside (products q * k are exact in fp64; w * max(0, d) is
 * rounded, then added), rounded once to fp32, -0 stored as +0: the exact
 * value the decode step's selection orders by.  n_idx_heads in [1, 64];
 * n_rows in [0, CSA_MAX_ROWS]; idx_rows and q_idx must be 16-byte aligned
 * (CSA_EINVAL otherwise); ws sized by csa_workspace_bytes(n_rows, 1).  The
 * fp64 arithmetic bounds this call (about 0.2 ms per million rows at 64
 * heads); the decode step scores exactly only the rows its filter cannot
 * place (csa_score_bounds). */
int csa_score(const uint8_t *idx_rows, int64_t n_rows, const float *q_idx, const float *w_idx,
              int n_idx_heads, float *scores, void *ws, size_t ws_bytes, void *hip_stream);

/* Exact top-k of a score array (DS4X page, "CSA score/top-512 fusion"):
 * the min(k, n_rows) largest scores, larger score first, equal scores by
 * lower row index, NaN after every number.  sel_idx[k] receives the rows
 * (-1 after the first min(k, n_rows)), sel_score[k] (may be NULL) their
 * scores (-inf padding).  k in [1, 512]. */
int csa_topk(const float *scores, int64_t n_rows, int k, int32_t *sel_idx, float *sel_score,
             void *ws, size_t ws_bytes, void *hip_stream);

/* Softmax attention over selected KV rows (DS4X page, kernel group "indexed
 * attention"; packed row layout from "Packed cache ABI").  Each selected row
 * is decoded to 512 fp32 values and serves as both key and value:
 *   l[h][t] = softmax_scale * q_attn[h] . kv[sel_idx[t]],
 *   out[h]  = sum_t softmax(l[h])[t] * kv[sel_idx[t]],
 *   lse[h]  = log(sum_t exp(l[h][t])).
 * n_sel in [0, 512] (n_sel = 0 gives out = 0 and lse = -inf); n_heads in
 * [1, 64]; lse may be NULL.  Entries of sel_idx outside [0, n_rows) are
 * skipped (they contribute nothing; with none valid, out = 0 and lse = -inf).
 * The logits and the value sum run on the bf16 matrix cores with exact
 * operand splits (query: three bf16 terms; weights: two; values exact, FP16
 * RoPE values as two terms), so products are exact and sums fp32. */
int csa_sparse_attn(const uint8_t *kv_rows, int64_t n_rows, const int32_t *sel_idx, int n_sel,
                    const float *q_attn, int n_heads, float softmax_scale, float *out, float *lse,
                    void *ws, size_t ws_bytes, void *hip_stream);

/* Rows accepted by csa_dense_attn. */
#define CSA_DENSE_MAX_ROWS (((int64_t)1) << 17)

/* Workspace bytes of csa_dense_attn over n_rows rows (0 if n_rows is out of
 * range). */
size_t csa_dense_workspace_bytes(int64_t n_rows);

/* Dense softmax attention over every KV row (the HCA layers of the DS4X page,
 * "What DS4X changes" and "Optimization details": exact score-split attention
 * over all compressed rows, with no row ceiling; at a 1M-token context a
 * ratio-128 layer holds 8,194 rows):
 *   l[h][j] = softmax_scale * q_attn[h] . kv[j]   for every row j < n_rows,
 *   out[h]  = sum_j softmax(l[h])[j] * kv[j],   lse[h] = log(sum_j exp(l[h][j])),
 * kv[j] the decoded 512-value row (csa_sparse_attn's operands and
 * arithmetic).  The rows are split into at most 256 contiguous groups of a
 * multiple of 32 rows whose partials are merged in group order.  n_rows in
 * [0, CSA_DENSE_MAX_ROWS] (n_rows = 0 gives out = 0 and lse = -inf); n_heads
 * in [1, 64]; lse may be NULL; ws sized by csa_dense_workspace_bytes(n_rows),
 * 256-byte aligned. */
int csa_dense_attn(const uint8_t *kv_rows, int64_t n_rows, const float *q_attn, int n_heads, float softmax_scale,
                   float *out, float *lse, void *ws, size_t ws_bytes, void *hip_stream);

/* Multi-token score and exact top-k over one history (DS4X page, "Packed
 * prefill implementation": batch score/top-k for several query tokens, as in
 * prefill and speculative verification): for every token t < n_tokens, the
 * exact top-k of csa_score over idx_rows with query q_idx + t*n_idx_heads*128
 * and weights w_idx + t*n_idx_heads (csa_topk order), written to
 * sel_idx + t*k and, if sel_score is not NULL, sel_score + t*k.  Each
 * token's selection is bit-identical to csa_score -> csa_topk for that
 * token; the tokens' score passes run tile by tile side by side so a tile's
 * rows are read from HBM once for all of them.  n_tokens in [1, 64],
 * n_idx_heads in [1, 64], k in [1, 512]; idx_rows and q_idx 16-byte aligned;
 * ws sized by csa_workspace_bytes(n_rows, n_tokens). */
int csa_score_topk_multi(const uint8_t *idx_rows, int64_t n_rows, const float *q_idx, const float *w_idx,
                         int n_tokens, int n_idx_heads, int k, int32_t *sel_idx, float *sel_score, void *ws,
                         size_t ws_bytes, void *hip_stream);

/* New rows in the packed formats (DS4X page, "Packed cache ABI": new
 * compressed rows and raw sliding-window ring rows are stored as 583-byte KV
 * rows, compressed indexer keys as 68-byte rows).  Row j of kv_vals
 * ([n_rows][512] fp32: 448 non-RoPE values, then 64 RoPE values) is written
 * to kv_rows + 583 j, row j of idx_vals ([n_rows][128]) to idx_rows + 68 j;
 * either value array may be NULL (that output is not written), not both.
 * The pages name the formats but not the conversion; this is the OCP MX v1.0
 * block conversion: per block the UE8M0 byte is floor(log2 max|v|) - emax +
 * 127 (emax 8 for E4M3 over 64 values, 2 for E2M1 over 32) clamped to
 * [0, 254], 127 for an all-zero block; each element v / 2^(byte-127) rounds
 * to the nearest element value, ties to the even significand, saturating at
 * 448 / 6, a value rounding to zero stored as +0; RoPE values become IEEE
 * binary16 (round to nearest even, overflow to infinity).  Inputs must be
 * finite.  kv_vals 4-byte and idx_vals 8-byte aligned; n_rows in
 * [0, CSA_MAX_ROWS]. */
int csa_pack_rows(const float *kv_vals, const float *idx_vals, int64_t n_rows, uint8_t *kv_rows, uint8_t *idx_rows,
                  void *hip_stream);

/* Merge of two attention results over disjoint row sets into the attention
 * over their union (the sliding-window raw ring and the selected compressed
 * rows in one softmax): with a = lse_a[h], b = lse_b[h], M = max(a, b),
 *   out[h] = (e^{a-M} out_a[h] + e^{b-M} out_b[h]) / (e^{a-M} + e^{b-M}),
 *   lse[h] = M + log(e^{a-M} + e^{b-M});
 * a side with lse = -inf (no row) weighs nothing; both -inf give out = 0 and
 * lse = -inf.  All arrays [n_heads][512] / [n_heads], n_heads in [1, 64];
 * out may be out_a or out_b (in place), lse must not be lse_a or lse_b. */
int csa_lse_merge(const float *out_a, const float *lse_a, const float *out_b, const float *lse_b, int n_heads,
                  float *out, float *lse, void *hip_stream);

/* One CSA decode step for each of n_sessions independent sessions: score
 * every indexer row, select the exact top-512 (csa_topk order) and attend
 * over the selected KV rows (csa_sparse_attn).  Selections and outputs are
 * bit-identical to csa_score -> csa_topk(k = 512) -> csa_sparse_attn on the
 * same inputs.  `sessions` is a HOST array; n_sessions in [1, 64];
 * n_idx_heads, n_heads in [1, 64]; ws sized by csa_workspace_bytes for the
 * largest session. */
int csa_decode_step(const csa_session *sessions, int n_sessions, int n_idx_heads, int n_heads,
                    float softmax_scale, void *ws, size_t ws_bytes, void *hip_stream);

/* Stages of csa_decode_step, in launch order: 0 filter score + tile heads,
 * 1 exact rescoring of the candidates, 2 selection + attention partials,
 * 3 merge of the partials. */
#define CSA_STAGES 4

/* csa_decode_step that also records events[2*s] right before and
 * events[2*s+1] right after the launches of stage s on hip_stream, so a
 * caller can time each stage with hipEventElapsedTime; stage 0's score
 * kernel records its two events at its own start and end (an extended HIP
 * launch), so they time the kernel rather than the queue around it.
 * `events` is a HOST array of 2*CSA_STAGES hipEvent_t (as void*) created by
 * the caller; the work done is exactly that of csa_decode_step. */
int csa_decode_step_timed(const csa_session *sessions, int n_sessions, int n_idx_heads, int n_heads,
                          float softmax_scale, void *ws, size_t ws_bytes, void *hip_stream,
                          void *const *events);

/* csa_decode_step with a choice of indexer query format (CSA_QUERY_FP32 or
 * CSA_QUERY_MXFP4; any other value gives CSA_EINVAL) and optional stage
 * events (NULL, or 2*CSA_STAGES events as for csa_decode_step_timed).  With
 * CSA_QUERY_MXFP4 each session's q_idx is quantized as csa_quantize_query
 * does, and the selection is the exact top-512 of csa_score over the decoded
 * quantized query (csa_dequant_idx of csa_quantize_query's rows): selections
 * and sel_score are bit-identical to csa_quantize_query -> csa_dequant_idx ->
 * csa_score -> csa_topk(k = 512).  The attention is unchanged.  Other
 * arguments and rules as csa_decode_step. */
int csa_decode_step_ex(const csa_session *sessions, int n_sessions, int n_idx_heads, int n_heads,
                       float softmax_scale, int query_format, void *ws, size_t ws_bytes, void *hip_stream,
                       void *const *events);

/* MXFP4 quantization of an indexer query q_idx [n_idx_heads][128] (device,
 * 16-byte aligned) into q_rows [n_idx_heads][68] (device, 4-byte aligned),
 * packed like indexer rows.  The pages do not say how their MXFP4 scorer
 * quantizes the query; this is the OCP MX v1.0 conversion of each 32-value
 * block: the UE8M0 byte is floor(log2 max|v|) - 2 + 127, clamped at 0 (0 for
 * an all-zero block), and each element is v / 2^(byte-127) rounded to the
 * nearest E2M1 value, ties to the even code, magnitudes past 6 saturating
 * to 6, sign kept (a negative value that rounds to zero gives -0).  Inputs
 * must be finite.  n_idx_heads in [1, 64]. */
int csa_quantize_query(const float *q_idx, int n_idx_heads, uint8_t *q_rows, void *hip_stream);

/* Bytes of the library's static per-device workspace (csa_decode_step_noalloc). */
#define CSA_SCRATCH_BYTES (32u << 20)

/* csa_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static array of
 * CSA_SCRATCH_BYTES in the library's device code: each GPU the library runs
 * on holds its own copy from the module's load until the process ends.  The
 * call allocates nothing (no hipMalloc, no allocating library routine); the
 * caller still owns every input and output.  Returns CSA_EWORKSPACE, with
 * nothing enqueued, when csa_workspace_bytes(largest n_rows, n_sessions)
 * exceeds CSA_SCRATCH_BYTES (1,048,576 rows in one session fit).  Results
 * are bit-identical to csa_decode_step.  All calls on one GPU share its
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller; the array keeps the last call's
 * contents, which no call reads before writing. */
int csa_decode_step_noalloc(const csa_session *sessions, int n_sessions, int n_idx_heads, int n_heads,
                            float softmax_scale, void *hip_stream);

/* Test entry point: the decode step's matrix-core filter.  For every row,
 * lower[j] <= scores[j] <= upper[j], scores as csa_score computes them (with
 * CSA_QUERY_MXFP4: over the decoded quantized query).  The filter scores the
 * row on the block-scaled matrix cores, with the query held to three fp6
 * terms per 32-value block (CSA_QUERY_FP32) or as its one MXFP4 operand, and
 * brackets the exact score by a rigorous bound from the query's residual and
 * term magnitudes, the head weights and the row's four UE8M0 bytes (a byte
 * >= 253 gives an infinite bracket).  Same arguments and rules as csa_score;
 * query_format as for csa_decode_step_ex. */
int csa_score_bounds(const uint8_t *idx_rows, int64_t n_rows, const float *q_idx, const float *w_idx,
                     int n_idx_heads, int query_format, float *upper, float *lower, void *ws, size_t ws_bytes,
                     void *hip_stream);

/* Test entry points: decode packed rows to fp32, [n][128] and [n][512]
 * (exact products; overflow gives +-inf; a 0xFF scale or an E4M3 NaN code
 * gives NaN).  Used to check the kernels' decode bit for bit. */
int csa_dequant_idx(const uint8_t *idx_rows, int64_t n_rows, float *out, void *hip_stream);
int csa_dequant_kv(const uint8_t *kv_rows, int64_t n_rows, float *out, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
