/* csa_gen.h -- seeded synthetic inputs for the CSA decode step (test and bench
 * infrastructure; holds no decode/score/select/attention arithmetic). */
#ifndef CSA_GEN_H
#define CSA_GEN_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

uint64_t csa_gen_seed(int config_id);
uint64_t csa_gen_u64(uint64_t seed, uint64_t stream, uint64_t i);
float csa_gen_normal(uint64_t seed, uint64_t stream, uint64_t i);
float csa_gen_uniform(uint64_t seed, uint64_t stream, uint64_t i);

/* Encoders: 128 fp32 -> one 68-byte indexer row; 512 fp32 -> one 583-byte KV row. */
void csa_gen_pack_idx_row(const float *v, uint8_t *row);
void csa_gen_pack_kv_row(const float *v, uint8_t *row);
uint16_t csa_gen_f16_bits(float x);
uint8_t csa_gen_e4m3_bits(double x);

/* Rows row0 .. row0+n-1 of one session's history (prefix-stable). */
void csa_gen_idx_rows(uint64_t seed, int session, int64_t row0, int64_t n, uint8_t *out);
void csa_gen_kv_rows(uint64_t seed, int session, int64_t row0, int64_t n, uint8_t *out);
/* q_idx [n_idx_heads][128] N(0,1), w_idx [n_idx_heads] U(0,1), q_attn [n_heads][512] N(0,1). */
void csa_gen_queries(uint64_t seed, int session, int n_idx_heads, int n_heads, float *q_idx,
                     float *w_idx, float *q_attn);
uint64_t csa_gen_fnv1a64(const void *p, int64_t n);

#ifdef __cplusplus
}
#endif
#endif
