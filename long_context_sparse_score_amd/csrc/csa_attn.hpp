// csa_attn.hpp -- attention logits of selected KV rows on the gfx950 bf16
// matrix cores (V_MFMA_F32_16X16X32_BF16), shared by the fused selection
// kernel and the stand-alone logits kernel so both give identical values.
//
// l[h][j] = scale * sum_d q[h][d] * kv_j[d] (DS4X page, "Packed cache ABI"
// for the row; the decoded 512-value row is both key and value).  Every
// operand enters exactly:
//   * a decoded non-RoPE value is an E4M3 value times 2^(s-127): at most 4
//     significant bits, exact in bf16;
//   * a RoPE value is FP16 (11 bits): hi = bf16(v), lo = v - hi (exact, <= 3
//     bits), two bf16 terms;
//   * the fp32 query is q0 + q1 + q2 with q_t = bf16(q - q0 - ... - q_{t-1})
//     (round to nearest even), leaving a residual below 2^-26 |q|.
// Products of bf16 values are exact in fp32 and accumulate in fp32.  The
// value of l[h][j] depends only on head h and row j, never on the other rows
// of the batch.
//
// Lane layout of the 16x16x32 instruction (verified on MI355X): lane l holds
// A[m = l%16][k = 8(l/16) .. +8) and B[k = 8(l/16) .. +8][n = l%16]; the
// result gives lane l C[m = 4(l/16) + v][n = l%16], v < 4.  Here m = head,
// n = row, k = dimension.  The 1024 threads of a workgroup are 16 waves:
// wave w takes head group g = w%4 (heads 16g..16g+15) and the dimension
// quarter kq = w/4 (dimensions 128kq..128kq+127, four K steps of 32); the
// four quarters are summed in order through LDS.
#pragma once

#include "../../include/csa.h"
#include "csa_device.hpp"

namespace csa {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f_attn __attribute__((ext_vector_type(4)));

constexpr int kKvDim = 512;
constexpr int kLogitThreads = 1024;
constexpr int kLogitRows = 16;  // rows per matrix-core batch
constexpr int kKvLdsStride = kKvDim + 4;

struct LogitShared {
  float kv[kLogitRows][kKvLdsStride];  // decoded rows of the batch
  float red[4][4][64][4];              // [quarter][head group][lane][v] partials
  int32_t row[kLogitRows];             // KV row, or -1 (the logit is -inf)
  int32_t pos[kLogitRows];             // output column (rank / position)
};

// This lane's query terms: K step s of its quarter, term t.
struct LogitQuery {
  v8bf a[4][3];
};

__device__ __forceinline__ void split3_bf16(float x, __bf16 &t0, __bf16 &t1, __bf16 &t2) {
  t0 = (__bf16)x;
  const float r1 = x - (float)t0;
  t1 = (__bf16)r1;
  t2 = (__bf16)(r1 - (float)t1);
}

// Raw query values of this lane: q[16g + l%16][128kq + 32s + 8(l/16) + i].
struct LogitQueryRaw {
  float v[4][8];
};

__device__ __forceinline__ void load_logit_query(LogitQueryRaw &r, const float *__restrict__ q_attn, int n_heads) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = wave & 3, kq = wave >> 2;
  const int h = 16 * g + (lane & 15);
  const float *src = q_attn + (size_t)h * kKvDim + 128 * kq + 8 * (lane >> 4);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[s][i] = (h < n_heads) ? src[32 * s + i] : 0.0f;
}

__device__ __forceinline__ void split_logit_query(LogitQuery &q, const LogitQueryRaw &r) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __bf16 t0, t1, t2;
      split3_bf16(r.v[s][i], t0, t1, t2);
      q.a[s][0][i] = t0;
      q.a[s][1][i] = t1;
      q.a[s][2][i] = t2;
    }
}

// The two bytes that determine decoded value i of a packed KV row (code and
// block scale, or the two bytes of an FP16 RoPE value), and the value from
// them.  Callers load the bytes of all their values first and decode after,
// so the loads are in flight together.
__device__ __forceinline__ void kv_load(const uint8_t *__restrict__ p, int i, uint32_t &b0, uint32_t &b1) {
  const bool nope = i < kKvNope;
  const int t = 2 * (i - kKvNope);
  b0 = p[nope ? i : kKvNope + t];
  b1 = p[nope ? kKvNope + 128 + (i >> 6) : kKvNope + t + 1];
}
__device__ __forceinline__ float kv_decode(int i, uint32_t b0, uint32_t b1) {
  const float vn = e4m3_value(b0) * ue8m0_scale(b1);
  const float vr = f16_value(b0 | (b1 << 8));
  return i < kKvNope ? vn : vr;
}

// Decode the rows sh.row[0..nb) into sh.kv (0 for rows < 0 and past nb).
// Invalid rows read row 0 and discard it; have_rows = false (an empty
// history, possibly no buffer) skips every load.  All kLogitThreads threads
// call it.
__device__ __forceinline__ void decode_logit_rows(const uint8_t *__restrict__ kv_rows, bool have_rows,
                                                  LogitShared &sh, int nb) {
  constexpr int U = kLogitRows * kKvDim / kLogitThreads;
  uint32_t b0[U], b1[U];
  int32_t row[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e = threadIdx.x + kLogitThreads * u;
    const int r = e / kKvDim;
    row[u] = r < nb ? sh.row[r] : -1;
  }
  if (have_rows) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = threadIdx.x + kLogitThreads * u;
      kv_load(kv_rows + (size_t)(uint32_t)max(row[u], 0) * kKvRowBytes, e % kKvDim, b0[u], b1[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e = threadIdx.x + kLogitThreads * u;
    const float x = have_rows ? kv_decode(e % kKvDim, b0[u], b1[u]) : 0.0f;
    sh.kv[e / kKvDim][e % kKvDim] = row[u] >= 0 ? x : 0.0f;
  }
}

// logits[h * 512 + sh.pos[n]] for rows n < nb and heads h < n_heads (rows
// with sh.row[n] < 0 get -inf).  sh.kv must hold the decoded batch; all
// kLogitThreads threads call it; it ends with a barrier.
__device__ __forceinline__ void batch_logits(const LogitQuery &q, LogitShared &sh, int nb, int n_heads,
                                             float scale, float *__restrict__ logits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = wave & 3, kq = wave >> 2;
  v4f_attn c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float *src = &sh.kv[lane & 15][128 * kq + 32 * s + 8 * (lane >> 4)];
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = src[i];
    v8bf hi;
#pragma unroll
    for (int i = 0; i < 8; ++i) hi[i] = (__bf16)f[i];
#pragma unroll
    for (int t = 0; t < 3; ++t) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q.a[s][t], hi, c, 0, 0, 0);
    if (kq == 3 && s >= 2) {  // RoPE dimensions 448..511: the FP16 remainder
      v8bf lo;
#pragma unroll
      for (int i = 0; i < 8; ++i) lo[i] = (__bf16)(f[i] - (float)hi[i]);
#pragma unroll
      for (int t = 0; t < 3; ++t) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q.a[s][t], lo, c, 0, 0, 0);
    }
  }
  if (kq != 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) sh.red[kq][g][lane][v] = c[v];
  }
  __syncthreads();
  if (kq == 0) {
    const int n = lane & 15;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float sum = ((c[v] + sh.red[1][g][lane][v]) + sh.red[2][g][lane][v]) + sh.red[3][g][lane][v];
      const int h = 16 * g + 4 * (lane >> 4) + v;
      if (n < nb && h < n_heads)
        logits[(size_t)h * CSA_TOPK + sh.pos[n]] = sh.row[n] >= 0 ? scale * sum : -__builtin_inff();
    }
  }
  __syncthreads();
}

}  // namespace csa
