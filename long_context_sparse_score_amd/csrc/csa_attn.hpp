// csa_attn.hpp -- softmax attention over a group of selected KV rows on the
// gfx950 bf16 matrix cores (V_MFMA_F32_16X16X32_BF16), the flash-decoding
// split used by both the fused selection kernel and csa_sparse_attn.
//
// The selected rows are partitioned into kAttnGroups fixed groups by a hash
// of the row index; a workgroup takes one group, visits its rows in rank
// (position) order, 32 at a time, and keeps for every head h
//   m_h = max logit seen, l_h = sum exp(l - m_h), acc_h[d] = sum exp(l - m_h) kv[d]
// (rescaled when m_h grows).  It writes (m, l, acc) as the group's partial;
// attn_combine merges the groups:
//   out[h] = sum_b e^{m_b - M} acc_b / sum_b e^{m_b - M} l_b,
//   lse[h] = M + log sum_b e^{m_b - M} l_b,   M = max_b m_b.
// Logits l[h][j] = scale * q_h . kv_j and values use the decoded 512-value
// row for both (DS4X page, "Packed cache ABI").  Every operand enters the
// matrix cores exactly:
//   * a decoded non-RoPE value is an E4M3 value times 2^(s-127): at most 4
//     significant bits, one bf16 term (exact for magnitudes >= 2^-133);
//   * a RoPE value is FP16 (11 bits): hi = bf16(v), lo = v - hi, two terms;
//   * the fp32 query is q0 + q1 + q2, q_t = bf16(q - q0 - ... - q_{t-1})
//     (round to nearest even), residual below 2^-26 |q|; it is split once
//     per call by the query-split kernel;
//   * a softmax weight p in [0, 1] is hi + lo (two bf16 terms, residual
//     below 2^-17 p).
// Products of bf16 values are exact in fp32; sums are fp32.  Everything a
// group computes depends only on its rows and their order, so the fused and
// the stand-alone paths give identical bits.
//
// Lane layout of the 16x16x32 instruction (verified on MI355X): lane l holds
// A[m = l%16][k = 8(l/16) .. +8) and B[k = 8(l/16) .. +8][n = l%16]; the
// result gives lane l C[m = 4(l/16) + v][n = l%16], v < 4.
// A workgroup is 8 waves; wave w takes head group g = w%4 (heads
// 16g..16g+15) and half hv = w/4:
//   logits: m = head, n = row, k = dimension; the wave covers dimension
//           quarters 2hv and 2hv+1 (four K steps of 32 each) for the two
//           16-row tiles of the batch; per row the four quarters are summed
//           as (q0 + q1) + (q2 + q3), the pairs meeting in LDS.
//   P V:    m = head, n = dimension, k = row (the batch's 32 rows); the
//           wave covers the 128 dimensions of chunks 2hv
//           and 2hv+1 (eight 16-wide tiles each).
#pragma once

#include "../../include/csa.h"
#include "csa_device.hpp"

namespace csa {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f_attn __attribute__((ext_vector_type(4)));

constexpr int kKvDim = 512;
constexpr int kAttnThreads = 512;
constexpr int kAttnGroups = 32;
constexpr int kAttnBatch = 32;  // rows per matrix-core batch (the K of the P V product)
constexpr int kKvLdsStride = kKvDim + 4;

// Group of a selected row (also the workgroup of the fused selection that
// ranks it): the top 5 bits of a multiplicative hash.
__device__ __forceinline__ uint32_t attn_group(uint32_t row) { return (row * 0x9E3779B1u) >> 27; }

// Attention query split in the workspace, per session:
// [g + 4 kq][K step 4][term 3][lane 64] x 8 bf16 (16 bytes).
constexpr int kAttnQVecs = 16 * 4 * 3 * 64;
constexpr size_t kAttnQBytes = (size_t)kAttnQVecs * 16;
// Partials per session: acc [group][head][512] and (m, l) [group][head][2].
constexpr size_t kAttnPartFloats = (size_t)kAttnGroups * CSA_MAX_HEADS * kKvDim;
constexpr size_t kAttnMlFloats = (size_t)kAttnGroups * CSA_MAX_HEADS * 2;

__device__ __forceinline__ size_t attn_q_index(int wave, int s, int t, int lane) {
  return ((size_t)(wave * 4 + s) * 3 + t) * 64 + lane;
}

// Packed rows staged in LDS, realigned: slot i holds its row's 583 bytes
// from byte 0.
constexpr int kRawStride = 592;  // bytes per slot: 148 dwords
constexpr int kRawRows = 32;     // rows staged at once

struct AttnStage {
  float kv[kAttnBatch][kKvLdsStride];       // decoded rows of the batch
  float lg[CSA_MAX_HEADS][kAttnBatch + 1];  // logits of the batch
  float red[2][4][64][4];                   // half-sums of the logits [half][g]
  int32_t row[kAttnBatch];                  // KV row, or -1 (padding)
  uint32_t raw[kRawRows][kRawStride / 4];   // staged packed rows
};

// x = t0 + t1 + t2 + r: three bf16 terms, each the round-to-nearest-even of
// what the previous ones leave (the subtractions are exact in fp32).
__device__ __forceinline__ void split3_bf16(float x, __bf16 &t0, __bf16 &t1, __bf16 &t2) {
  t0 = (__bf16)x;
  const float r1 = x - (float)t0;
  t1 = (__bf16)r1;
  t2 = (__bf16)(r1 - (float)t1);
}

// Split task t < kAttnQVecs / 3 of a session's attention query q[n][512]
// (n = n_heads; heads past n are zero): the three terms of
//   q[16(w%4) + l%16][128(w/4) + 32s + 8(l/16) + i], i < 8,
// for w = t / 256, s = (t / 64) % 4, l = t % 64, stored at
// dst[attn_q_index(w, s, term, l)].
__device__ __forceinline__ void attn_q_split_task(const float *__restrict__ qa, int n_heads, uint4 *__restrict__ dst,
                                                  int t) {
  const int lane = t % 64, s = (t / 64) % 4, wave = t / 256;
  const int h = 16 * (wave & 3) + (lane & 15);
  const int d0 = 128 * (wave >> 2) + 32 * s + 8 * (lane >> 4);
  const bool live = h < n_heads;
  const float *src = qa + (size_t)(live ? h : 0) * kKvDim + d0;
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = src[i];
    x[i] = live ? v : 0.0f;
  }
  v8bf t0, t1, t2;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __bf16 a0, a1, a2;
    split3_bf16(x[i], a0, a1, a2);
    t0[i] = a0;
    t1[i] = a1;
    t2[i] = a2;
  }
  dst[attn_q_index(wave, s, 0, lane)] = __builtin_bit_cast(uint4, t0);
  dst[attn_q_index(wave, s, 1, lane)] = __builtin_bit_cast(uint4, t1);
  dst[attn_q_index(wave, s, 2, lane)] = __builtin_bit_cast(uint4, t2);
}
constexpr int kAttnQTasks = kAttnQVecs / 3;  // 4096

// This lane's query terms: quarter 2hv + kl, K step s, term t.
struct AttnQuery {
  v8bf a[2][4][3];
};

__device__ __forceinline__ void load_attn_query(AttnQuery &q, const uint4 *qs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = wave & 3, hv = wave >> 2;
#pragma unroll
  for (int kl = 0; kl < 2; ++kl)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const uint4 v = qs[attn_q_index(g + 4 * (2 * hv + kl), s, t, lane)];
        q.a[kl][s][t] = __builtin_bit_cast(v8bf, v);
      }
}

// Per-wave state of a group: accumulator tiles (heads 16g + 4(l/16) + v,
// dimensions 128(2hv + cl) + 16t + l%16) and the running max / sum of head
// 16g + l%16.
struct AttnState {
  v4f_attn acc[2][8];
  float m, l;
};

__device__ __forceinline__ void attn_init(AttnState &S) {
#pragma unroll
  for (int cl = 0; cl < 2; ++cl)
#pragma unroll
    for (int t = 0; t < 8; ++t) S.acc[cl][t] = v4f_attn{0.0f, 0.0f, 0.0f, 0.0f};
  S.m = -__builtin_inff();
  S.l = 0.0f;
}

// Stage rows[0..m) (valid KV row indices, m <= kRawRows) into st.raw: slot
// i receives row rows[i]'s bytes from byte 0 (146 dwords).  Lane j of the
// wave builds dwords j, j + 64, j + 128 of a row from the two aligned dwords
// that hold them (v_alignbyte); only dwords holding a byte of the row are
// read, so nothing past the buffer's last byte is touched.  Wave w copies
// rows w, w + 8, ..., two rows per pass, all loads first.  All threads call
// it; the caller synchronizes before reading the slots.
constexpr int kRawDwords = (kKvRowBytes + 3) / 4;  // 146
__device__ __forceinline__ void attn_stage_raw(const uint8_t *__restrict__ kv_rows, const int32_t *rows, int m,
                                               AttnStage &st) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int kWaves = kAttnThreads / 64;
  constexpr int kPass = 2;
  for (int i0 = wave; i0 < m; i0 += kPass * kWaves) {
    uint32_t lo[kPass][3], hi[kPass][3], sh[kPass];
#pragma unroll
    for (int u = 0; u < kPass; ++u) {
      const int i = i0 + kWaves * u;
      const int32_t r = __builtin_amdgcn_readfirstlane(rows[i < m ? i : i0]);
      const uint8_t *rb = kv_rows + (size_t)(uint32_t)r * kKvRowBytes;
      const uint32_t mis = (uint32_t)(uintptr_t)rb & 3u;
      const uint32_t *a0 = reinterpret_cast<const uint32_t *>(rb - mis);  // stays a global pointer
      const int last = (int)(mis + kKvRowBytes - 1) >> 2;                 // dword of the last byte
      sh[u] = 8u * mis;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int j = lane + 64 * k;
        lo[u][k] = a0[j < last ? j : last];  // clamped: no branch around the loads
        hi[u][k] = a0[j + 1 < last ? j + 1 : last];
      }
    }
#pragma unroll
    for (int u = 0; u < kPass; ++u) {
      const int i = i0 + kWaves * u;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int j = lane + 64 * k;
        const uint32_t w = (uint32_t)(((uint64_t)hi[u][k] << 32 | lo[u][k]) >> sh[u]);
        if (i < m && j < kRawDwords) st.raw[i][j] = w;
      }
    }
  }
}

// One batch: rows st.row[0..kAttnBatch) (-1 = padding) are decoded into
// st.kv, their logits go to st.lg, and this wave's running softmax state and
// accumulators are updated.  All kAttnThreads threads call it; it starts and
// ends with a barrier.
__device__ __forceinline__ void attn_batch(const uint4 *qsplit, AttnState &S, AttnStage &st, int slot0,
                                           float scale) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __syncthreads();  // st.row written
  // the query terms (L2-resident, shared by every group) are loaded with the
  // rows' bytes and live only through the logits
  AttnQuery q;
  load_attn_query(q, qsplit);
  {
    // decode: 32 rows x 512 values in two passes of 16, all LDS reads of a
    // pass first.  Wave
    // w takes values [64w, 64w + 64) of every row (one per lane): waves 0..6
    // hold E4M3 values of one scale block per row, wave 7 the FP16 RoPE
    // values, so the branch is uniform.  The conversions are gfx950's
    // v_cvt_scalef32_f32_fp8 (code x scale, exact; checked on MI355X on all
    // 256 codes, scale bytes 0..255 included) and v_cvt_f32_f16 (exact).
    static_assert(kAttnThreads == kKvDim, "one value per lane and row");
    constexpr int U = 16;  // rows per pass
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int col = 64 * wv + lane;
#pragma unroll
    for (int u0 = 0; u0 < kAttnBatch; u0 += U) {
      const uint8_t *base = reinterpret_cast<const uint8_t *>(&st.raw[slot0 + u0][0]);
      float x[U];
      if (wv < kKvNope / 64) {
        uint32_t code[U], sb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          code[u] = base[u * kRawStride + col];
          sb[u] = base[u * kRawStride + kKvNope + 128 + wv];  // the block's scale byte (same in every lane)
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t e = __builtin_amdgcn_readfirstlane(sb[u]);
          x[u] = __builtin_amdgcn_cvt_scalef32_f32_fp8((int)code[u], ue8m0_scale(e), 0);
        }
      } else {
        uint32_t h[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          h[u] = *reinterpret_cast<const uint16_t *>(base + u * kRawStride + kKvNope + 2 * (col - kKvNope));
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = (float)__builtin_bit_cast(_Float16, (uint16_t)h[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t r = __builtin_amdgcn_readfirstlane(st.row[u0 + u]);
        st.kv[u0 + u][col] = r >= 0 ? x[u] : 0.0f;
      }
    }
  }
  __syncthreads();
  const int g = wave & 3, hv = wave >> 2;
  // logits of the batch's 32 rows (two 16-row tiles nt), this wave's two
  // dimension quarters; per row the four quarters are summed as
  // (q0 + q1) + (q2 + q3), wave half hv finishing row tile nt = hv
  v4f_attn cw[2];  // per row tile: quarters 2hv + 2hv+1
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    v4f_attn c[2];
#pragma unroll
    for (int kl = 0; kl < 2; ++kl) {
      const int kq = 2 * hv + kl;
      c[kl] = v4f_attn{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float *src = &st.kv[16 * nt + (lane & 15)][128 * kq + 32 * s + 8 * (lane >> 4)];
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = src[i];
        v8bf hi;
#pragma unroll
        for (int i = 0; i < 8; ++i) hi[i] = (__bf16)f[i];
#pragma unroll
        for (int t = 0; t < 3; ++t) c[kl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q.a[kl][s][t], hi, c[kl], 0, 0, 0);
        if (kq == 3 && s >= 2) {  // RoPE dimensions 448..511: the FP16 remainder
          v8bf lo;
#pragma unroll
          for (int i = 0; i < 8; ++i) lo[i] = (__bf16)(f[i] - (float)hi[i]);
#pragma unroll
          for (int t = 0; t < 3; ++t) c[kl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q.a[kl][s][t], lo, c[kl], 0, 0, 0);
        }
      }
    }
    cw[nt] = c[0] + c[1];
  }
  {
    const v4f_attn own = hv == 0 ? cw[0] : cw[1], other = hv == 0 ? cw[1] : cw[0];
#pragma unroll
    for (int v = 0; v < 4; ++v) st.red[hv][g][lane][v] = other[v];  // the partner's row tile
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float part = st.red[1 - hv][g][lane][v];
      const float sum = hv == 0 ? own[v] + part : part + own[v];  // (q0 + q1) + (q2 + q3)
      const int n = 16 * hv + (lane & 15);
      st.lg[16 * g + 4 * (lane >> 4) + v][n] = st.row[n] >= 0 ? scale * sum : -__builtin_inff();
    }
  }
  __syncthreads();
  // online softmax of this lane's head over the batch's rows: lane l holds
  // rows 8(l/16)..+8
  const int hh = 16 * g + (lane & 15);
  float pl[8];
  float mb = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pl[i] = st.lg[hh][8 * (lane >> 4) + i];
    mb = fmaxf(mb, pl[i]);
  }
  mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
  mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
  const float m_new = fmaxf(S.m, mb);
  const float mref = m_new == -__builtin_inff() ? 0.0f : m_new;
  const float alpha = __expf(S.m - mref);
  float ps = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pl[i] = __expf(pl[i] - mref);
    ps += pl[i];
  }
  ps += __shfl_xor(ps, 16, 64);
  ps += __shfl_xor(ps, 32, 64);
  S.l = S.l * alpha + ps;
  S.m = m_new;
  v8bf ph, plo;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ph[i] = (__bf16)pl[i];
    plo[i] = (__bf16)(pl[i] - (float)ph[i]);
  }
  // rescale the accumulators: element v of a tile is head 16g + 4(l/16) + v,
  // whose factor sits in lane 4(l/16) + v
  float av[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) av[v] = __shfl(alpha, 4 * (lane >> 4) + v, 64);
#pragma unroll
  for (int cl = 0; cl < 2; ++cl)
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) S.acc[cl][t][v] *= av[v];
  // acc += P V over the batch's 32 rows (the K of the product)
#pragma unroll
  for (int cl = 0; cl < 2; ++cl) {
    const int cc = 2 * hv + cl;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int d = 128 * cc + 16 * t + (lane & 15);
      v8bf vh, vl;
      float vf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        vf[i] = st.kv[8 * (lane >> 4) + i][d];
        vh[i] = (__bf16)vf[i];
      }
      S.acc[cl][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vh, S.acc[cl][t], 0, 0, 0);
      S.acc[cl][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, vh, S.acc[cl][t], 0, 0, 0);
      if (cc == 3 && t >= 4) {  // RoPE dimensions: the FP16 remainder
#pragma unroll
        for (int i = 0; i < 8; ++i) vl[i] = (__bf16)(vf[i] - (float)vh[i]);
        S.acc[cl][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vl, S.acc[cl][t], 0, 0, 0);
        S.acc[cl][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, vl, S.acc[cl][t], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // the stage is reused by the next batch
}

// Write the group's partial: acc [head][512] and (m, l) [head][2].
__device__ __forceinline__ void attn_store(const AttnState &S, int n_heads, float *__restrict__ part,
                                           float *__restrict__ ml) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = wave & 3, hv = wave >> 2;
  if (16 * g + 15 < n_heads) {  // every head of the wave exists (uniform)
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int h = 16 * g + 4 * (lane >> 4) + v;
          part[(size_t)h * kKvDim + 128 * (2 * hv + cl) + 16 * t + (lane & 15)] = S.acc[cl][t][v];
        }
  } else if (16 * g < n_heads) {
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int h = 16 * g + 4 * (lane >> 4) + v;
          if (h < n_heads) part[(size_t)h * kKvDim + 128 * (2 * hv + cl) + 16 * t + (lane & 15)] = S.acc[cl][t][v];
        }
  }
  const int hh = 16 * g + (lane & 15);
  if (hv == 0 && lane < 16 && hh < n_heads) {
    ml[2 * hh] = S.m;
    ml[2 * hh + 1] = S.l;
  }
}

// Merge of the group partials of one output element e = h * 512 + d:
//   out = sum_b e^{m_b - M} acc_b / sum_b e^{m_b - M} l_b,  M = max_b m_b,
//   lse = M + log sum_b e^{m_b - M} l_b
// (groups with m = -inf are empty and add nothing; with no row at all,
// out = 0 and lse = -inf).  ml, part: one session's partials.
__device__ __forceinline__ float attn_merge_element(const float *ml, const float *part, int h, int e, float &lse) {
  float mb[kAttnGroups], lb[kAttnGroups], xb[kAttnGroups];
#pragma unroll
  for (int b = 0; b < kAttnGroups; ++b) {
    mb[b] = ml[((size_t)b * CSA_MAX_HEADS + h) * 2];
    lb[b] = ml[((size_t)b * CSA_MAX_HEADS + h) * 2 + 1];
    xb[b] = part[(size_t)b * CSA_MAX_HEADS * kKvDim + e];
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int b = 0; b < kAttnGroups; ++b) M = fmaxf(M, mb[b]);
  float L = 0.0f, X = 0.0f;
  if (M != -__builtin_inff()) {
#pragma unroll
    for (int b = 0; b < kAttnGroups; ++b) {
      const float w = mb[b] == -__builtin_inff() ? 0.0f : __expf(mb[b] - M);
      L += w * lb[b];
      X += mb[b] == -__builtin_inff() ? 0.0f : w * xb[b];
    }
  }
  lse = L > 0.0f ? M + logf(L) : -__builtin_inff();
  return L > 0.0f ? X / L : 0.0f;
}

// Order a group's entries by their key (rank or position, distinct),
// ascending: out_rows[i] = row of the i-th.  keys/rows[0..m) in LDS; all
// threads call it; ends with a barrier.
__device__ __forceinline__ void attn_order(const int32_t *keys, const int32_t *rows, int m, int32_t *out_rows) {
  for (int i = threadIdx.x; i < m; i += kAttnThreads) {
    const int32_t k = keys[i];
    int r = 0;
    for (int j0 = 0; j0 < m; j0 += 16) {
#pragma unroll
      for (int u = 0; u < 16; ++u) r += (j0 + u < m && keys[j0 + u] < k) ? 1 : 0;
    }
    out_rows[r] = rows[i];
  }
  __syncthreads();
}

// Attention over a group's rows (in order) -> its partial.  All threads
// call it.
__device__ __forceinline__ void attn_group_rows(const uint4 *qsplit, AttnStage &st, const int32_t *rows,
                                                int m,
                                                const uint8_t *__restrict__ kv_rows, float scale, int n_heads,
                                                float *__restrict__ part, float *__restrict__ ml) {
  AttnState S;
  attn_init(S);
  for (int b0 = 0; b0 < m; b0 += kAttnBatch) {
    const int slot0 = b0 & (kRawRows - 1);
    if (slot0 == 0)  // stage the next kRawRows rows (the previous batch ended with a barrier)
      attn_stage_raw(kv_rows, rows + b0, m - b0 < kRawRows ? m - b0 : kRawRows, st);
    if (threadIdx.x < kAttnBatch) st.row[threadIdx.x] = b0 + (int)threadIdx.x < m ? rows[b0 + threadIdx.x] : -1;
    // starts with a barrier: rows staged, st.row written
    attn_batch(qsplit, S, st, slot0, scale);
  }
  attn_store(S, n_heads, part, ml);
}

}  // namespace csa
