/* csa_oracle.h -- CPU reference of the CSA decode step.  TEST INFRASTRUCTURE
 * ONLY (tests, smoke check, benchmark CPU baseline); never part of the
 * product path.  Shares nothing with the HIP library. */
#ifndef CSA_ORACLE_H
#define CSA_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

double csa_oracle_e2m1(int code);  /* 0..15 */
double csa_oracle_e4m3(int code);  /* 0..255 */
double csa_oracle_ue8m0(int byte); /* 0..255 */
double csa_oracle_f16(int bits);   /* 0..65535 */

void csa_oracle_decode_idx_rows(const uint8_t *rows, int64_t n, float *out /* [n][128] */);
void csa_oracle_decode_kv_rows(const uint8_t *rows, int64_t n, float *out /* [n][512] */);
void csa_oracle_score(const uint8_t *idx_rows, int64_t n, const float *q_idx, const float *w_idx,
                      int n_idx_heads, float *scores);
int64_t csa_oracle_topk(const float *scores, int64_t n, int k, int32_t *sel, float *sel_score);
int csa_oracle_attention(const uint8_t *kv_rows, int64_t n_rows, const int32_t *sel, int n_sel,
                         const float *q_attn, int n_heads, double softmax_scale, float *out,
                         float *lse);
/* For each of n_tokens queries ([n_tokens][n_idx_heads][128], weights
 * [n_tokens][n_idx_heads]) its exact top-k over the same rows
 * (sel, sel_score: [n_tokens][k]). */
int csa_oracle_score_topk_multi(const uint8_t *idx_rows, int64_t n, const float *q_idx, const float *w_idx,
                                int n_tokens, int n_idx_heads, int k, int32_t *sel, float *sel_score);
/* Softmax attention over every row (each row once, in row order). */
int csa_oracle_dense_attention(const uint8_t *kv_rows, int64_t n_rows, const float *q_attn, int n_heads,
                               double softmax_scale, float *out, float *lse);
/* New rows packed into the 583-byte KV format ([n][512] values) and the
 * 68-byte indexer format ([n][128] values). */
void csa_oracle_pack_kv_rows(const float *v, int64_t n, uint8_t *rows);
void csa_oracle_pack_idx_rows(const float *v, int64_t n, uint8_t *rows);
/* The merge of two attention results over disjoint rows ([n_heads][512] and
 * [n_heads] each). */
void csa_oracle_lse_merge(const float *out_a, const float *lse_a, const float *out_b, const float *lse_b,
                          int n_heads, float *out, float *lse);
/* The indexer query [n_heads][128] quantized to MXFP4 rows [n_heads][68]. */
void csa_oracle_quantize_query(const float *q, int n_heads, uint8_t *rows);
int csa_oracle_decode_step(const uint8_t *idx_rows, const uint8_t *kv_rows, int64_t n_rows,
                           const float *q_idx, const float *w_idx, int n_idx_heads,
                           const float *q_attn, int n_heads, double softmax_scale, int k,
                           int32_t *sel, float *sel_score, float *out, float *lse);

#ifdef __cplusplus
}
#endif
#endif
