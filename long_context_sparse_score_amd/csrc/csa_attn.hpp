// csa_attn.hpp -- softmax attention over a group of selected KV rows on the
// gfx950 bf16 matrix cores, the flash-decoding split used by both the fused
// selection kernel and csa_sparse_attn.
//
// The selected rows are partitioned into kAttnGroups fixed row groups by a
// hash of the row index, and the 64 heads into kAttnHeadGroups groups of 16;
// a workgroup takes one (row group, head group) pair, visits the group's
// rows in rank (position) order, 16 at a time, and keeps for every head h
//   m_h = max logit seen, l_h = sum exp(l - m_h), acc_h[d] = sum exp(l - m_h) kv[d]
// (rescaled when m_h grows).  It writes (m, l, acc) as the row group's
// partial of its heads; attn_combine merges the row groups:
//   out[h] = sum_b e^{m_b - M} acc_b / sum_b e^{m_b - M} l_b,
//   lse[h] = M + log sum_b e^{m_b - M} l_b,   M = max_b m_b.
// Logits l[h][j] = scale * q_h . kv_j and values use the decoded 512-value
// row for both (DS4X page, "Packed cache ABI").  Every operand enters the
// matrix cores exactly:
//   * a non-RoPE value is an E4M3 code (at most 4 significant bits, exact in
//     bf16) times its block's power of two 2^(s-127).  The codes enter
//     unscaled, converted from the packed bytes by gfx950's fp8 conversion;
//     the power of two is applied outside the products: to a wave's partial
//     logits (one wave's K range is exactly one 64-value block, so the scale
//     is one per row there), and to the softmax weights of P V relative to a
//     running block exponent of the wave (below), so no decoded magnitude is
//     cut off by bf16's range;
//   * a RoPE value is FP16 (11 bits): hi = bf16(v), lo = v - hi, two terms;
//   * the fp32 query is q0 + q1 + q2, q_t = bf16(q - q0 - ... - q_{t-1})
//     (round to nearest even), residual below 2^-26 |q|; it is split once
//     per call (by the score kernel or the query-split kernel);
//   * a softmax weight is hi + lo (two bf16 terms, residual below 2^-17 of
//     it).  In the E4M3 waves the weight of row j is p_j 2^(s_j - E), E the
//     largest block scale byte the wave has met so far: the accumulator is
//     kept in units of 2^(E-127) (rescaled exactly when E grows) and
//     multiplied by 2^(E-127) when the partial is written.
// Products of bf16 values are exact in fp32; sums are fp32 in a fixed
// order.  Everything a workgroup computes depends only on its rows and their
// order, so the fused and the stand-alone paths give identical bits.
//
// Matrix-core shapes (lane layouts verified on MI355X):
//   logits  V_MFMA_F32_16X16X32_BF16 with M = 16 rows, N = 16 heads,
//           K = 32 dimensions: lane l holds A[row l%16][k 8(l/16) .. +8],
//           B[k 8(l/16) .. +8][head l%16] and receives C[rows 4(l/16) + v][head l%16];
//   P V     V_MFMA_F32_16X16X16_BF16 with M = 16 heads, N = 16 dimensions,
//           K = 16 rows: lane l holds A[head l%16][rows 4(l/16) .. +4] --
//           exactly the softmax weights it computed from its logits, so no
//           transpose is needed -- and B[rows 4(l/16) .. +4][dim l%16], and
//           receives C[heads 4(l/16) + v][dim l%16].
// A workgroup is 8 waves: wave w forms the logits' K steps 2w and 2w + 1
// (dimensions 64w .. 64w + 63) for all 16 rows and heads; the eight partial
// logit tiles meet in LDS and every wave sums them in the same fixed order,
// then runs the same softmax; for P V wave w owns dimensions 64w .. +64.
#pragma once

#include "../../include/csa.h"
#include "csa_device.hpp"
#include "csa_stream.hpp"

namespace csa {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f_attn __attribute__((ext_vector_type(4)));

typedef short v8s_attn __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf_attn __attribute__((ext_vector_type(2)));

constexpr int kKvDim = 512;
constexpr int kAttnThreads = 512;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kAttnGroupsLg = 5;
constexpr int kAttnGroups = 1 << kAttnGroupsLg;  // row groups (at most)
constexpr int kAttnHeadGroups = 4;  // 16 heads each
constexpr int kAttnSlices = kAttnGroups * kAttnHeadGroups;  // workgroups per session
constexpr int kAttnBatch = 32;      // rows per matrix-core batch
static_assert(kAttnWaves * 64 == kKvDim, "one 64-dimension block per wave");

// Row group of a selected row among 2^lg row groups (lg <= 5): the top lg
// bits of a multiplicative hash.  With lg = 5 it is also the workgroup of
// the fused selection that ranks the row.
__device__ __forceinline__ uint32_t attn_group(uint32_t row, int lg) {
  return lg == 0 ? 0u : (row * 0x9E3779B1u) >> (32 - lg);
}

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
constexpr int kRawRows = 32;     // rows staged at once (one batch)
static_assert(kRawRows % kAttnBatch == 0, "batches do not straddle a staging round");

typedef uint32_t AttnRawRow[kRawStride / 4];  // one staging slot

struct AttnStage {
  alignas(16) AttnRawRow raw[kRawRows];    // staged packed rows
  float lgp[kAttnWaves][2][4][64];         // partial logit tiles [wave][tile][v][lane]
  float lgf[2][4][64];                     // their sums [tile][v][lane]
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
// dst[attn_q_index(w, s, term, l)].  attn_q_load reads the task's eight
// values (a head past n_heads reads head 0), attn_q_store zeroes those of a
// head past n_heads, splits and stores them: a caller can issue the loads
// early and consume them late.
__device__ __forceinline__ bool attn_q_live(int n_heads, int t) {
  return 16 * ((t / 256) & 3) + ((t % 64) & 15) < n_heads;
}
__device__ __forceinline__ void attn_q_load(const float *__restrict__ qa, int n_heads, int t, float (&x)[8]) {
  const int lane = t % 64, s = (t / 64) % 4, wave = t / 256;
  const int h = 16 * (wave & 3) + (lane & 15);
  const int d0 = 128 * (wave >> 2) + 32 * s + 8 * (lane >> 4);
  const float *src = qa + (size_t)(h < n_heads ? h : 0) * kKvDim + d0;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = src[i];
}
__device__ __forceinline__ void attn_q_store(const float (&x)[8], int n_heads, uint4 *__restrict__ dst, int t) {
  const int lane = t % 64, s = (t / 64) % 4, wave = t / 256;
  const bool live = attn_q_live(n_heads, t);
  v8bf t0, t1, t2;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __bf16 a0, a1, a2;
    split3_bf16(live ? x[i] : 0.0f, a0, a1, a2);
    t0[i] = a0;
    t1[i] = a1;
    t2[i] = a2;
  }
  dst[attn_q_index(wave, s, 0, lane)] = __builtin_bit_cast(uint4, t0);
  dst[attn_q_index(wave, s, 1, lane)] = __builtin_bit_cast(uint4, t1);
  dst[attn_q_index(wave, s, 2, lane)] = __builtin_bit_cast(uint4, t2);
}
__device__ __forceinline__ void attn_q_split_task(const float *__restrict__ qa, int n_heads, uint4 *__restrict__ dst,
                                                  int t) {
  float x[8];
  attn_q_load(qa, n_heads, t, x);
  attn_q_store(x, n_heads, dst, t);
}
constexpr int kAttnQTasks = kAttnQVecs / 3;  // 4096

// This wave's query terms for head group g: K steps 2w and 2w + 1, three
// terms each, in the B operand layout of the logits (lane l: head 16g +
// l%16, dimensions 32 ks + 8(l/16) .. +8).
struct AttnQuery {
  v8bf b[2][3];
};

__device__ __forceinline__ void load_attn_query(AttnQuery &q, const uint4 *qs, int g) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ks = 2 * wave + j;
#pragma unroll
    for (int t = 0; t < 3; ++t)
      q.b[j][t] = __builtin_bit_cast(v8bf, qs[attn_q_index(g + 4 * (ks >> 2), ks & 3, t, lane)]);
  }
}

// Per-wave state of a workgroup: P V accumulator tiles (heads 4(l/16) + v of
// the head group, dimensions 64w + 4(l%16) + i) and the running max / sum of
// head l%16 (the same in every lane of that head and in every wave).
struct AttnState {
  v4f_attn acc[4];
  float m, l;
  int e;  // E4M3 waves: the accumulator's block exponent (scale byte); 0 until a row is met
};

__device__ __forceinline__ void attn_init(AttnState &S) {
#pragma unroll
  for (int i = 0; i < 4; ++i) S.acc[i] = v4f_attn{0.0f, 0.0f, 0.0f, 0.0f};
  S.m = -__builtin_inff();
  S.l = 0.0f;
  S.e = 0;
}

__device__ __forceinline__ short bf16_bits(float x) { return __builtin_bit_cast(short, (__bf16)x); }

// fp16 bits -> (bf16 hi, bf16 lo) with hi + lo == the fp16 value exactly.
__device__ __forceinline__ void f16_split(uint32_t h, short &hi, short &lo) {
  const float f = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  const __bf16 b = (__bf16)f;
  hi = __builtin_bit_cast(short, b);
  lo = bf16_bits(f - (float)b);
}

// Logits A operand of K step ks (dimensions 32 ks .. +32) for the row in
// slot `slot`: the lane's 8 values at dimensions 32 ks + 8(l/16) .. +8, as
// bf16 (lo: the RoPE remainder; zero for E4M3 steps).  E4M3 values are the
// unscaled codes (the block's power of two is applied to the products' sum
// by the caller).  Zero for a padding row.
__device__ __forceinline__ void attn_row_operand(const AttnRawRow *raw, int slot, int ks, bool valid, v8bf &hi,
                                                 v8bf &lo) {
  const int lane = threadIdx.x & 63;
  const uint8_t *rb = reinterpret_cast<const uint8_t *>(&raw[slot][0]);
  if (ks < kKvNope / 32) {
    const uint2 c = *reinterpret_cast<const uint2 *>(rb + 32 * ks + 8 * (lane >> 4));
    const v2bf_attn p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, false);
    const v2bf_attn p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, true);
    const v2bf_attn p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, false);
    const v2bf_attn p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, true);
    hi = v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    if (!valid) hi = v8bf{};
    lo = v8bf{};
  } else {
    const uint4 h4 = *reinterpret_cast<const uint4 *>(rb + kKvNope + 64 * (ks - kKvNope / 32) + 16 * (lane >> 4));
    const uint32_t w[4] = {h4.x, h4.y, h4.z, h4.w};
    short sh[8], sl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f16_split((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu, sh[i], sl[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hi[i] = valid ? __builtin_bit_cast(__bf16, sh[i]) : (__bf16)0.0f;
      lo[i] = valid ? __builtin_bit_cast(__bf16, sl[i]) : (__bf16)0.0f;
    }
  }
}

// Staging slot of row b0 + i of a group's ordered rows: slotmap[b0 + i], or
// (b0 + i) % kRawRows without a map; slot 0 for padding (i >= nvalid).
__device__ __forceinline__ int attn_slot(const int32_t *slotmap, int b0, int i, int nvalid) {
  if (i >= nvalid) return 0;
  return slotmap ? slotmap[b0 + i] : (b0 + i) % kRawRows;
}

// One batch: rows b0 .. b0 + 31 of the group's ordered rows, of which the
// first `nvalid` (1 <= nvalid <= 32) exist and the rest are padding; row
// b0 + i is staged in slot attn_slot(slotmap, b0, i, nvalid).  The logits are
// two 16-row tiles (the second skipped when nvalid <= 16).  P V takes all 32
// rows in one K = 32 product per 16-dimension tile: K index 8(l/16) + 4u + i
// is row 16u + 4(l/16) + i, which is where lane l holds that row's logit of
// head l%16.  Updates this wave's running softmax state and accumulators.
// All kAttnThreads threads call it; it ends with a barrier (the partial
// tiles and the staged rows are reused).
__device__ __forceinline__ void attn_batch(const AttnQuery &q, AttnState &S, AttnStage &st, const AttnRawRow *raw,
                                           const int32_t *slotmap, int b0, int nvalid, float scale) {
  // the lane offsets below are recomputed per batch rather than hoisted out
  // of the caller's loop, where they would only hold registers
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const bool two = nvalid > 16;  // uniform
  // partial logits of the rows x 16 heads over dimensions 64w .. +64
  v4f_attn c[2] = {v4f_attn{0.0f, 0.0f, 0.0f, 0.0f}, v4f_attn{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ks = 2 * wave + j;  // uniform
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && !two) break;
      v8bf hi, lo;
      attn_row_operand(raw, attn_slot(slotmap, b0, 16 * u + lr, nvalid), ks, 16 * u + lr < nvalid, hi, lo);
#pragma unroll
      for (int t = 0; t < 3; ++t) c[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, q.b[j][t], c[u], 0, 0, 0);
      if (ks >= kKvNope / 32) {
#pragma unroll
        for (int t = 0; t < 3; ++t) c[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, q.b[j][t], c[u], 0, 0, 0);
      }
    }
  }
  if (wave < kKvNope / 64) {  // uniform: this wave's K range is block `wave` of every row
    // c[u][v] is the sum for row 16u + 4(l/16) + v over unscaled codes: times
    // the row's 2^(s-127) (one rounding at most, in the fp32 subnormal range)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && !two) break;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = 16 * u + 4 * lg + v;
        const uint8_t *rr = reinterpret_cast<const uint8_t *>(&raw[attn_slot(slotmap, b0, i, nvalid)][0]);
        c[u][v] *= ue8m0_scale(rr[kKvNope + 128 + wave]);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) st.lgp[wave][0][v][lane] = c[0][v];
  if (two) {
#pragma unroll
    for (int v = 0; v < 4; ++v) st.lgp[wave][1][v][lane] = c[1][v];
  }
  __syncthreads();
  // the full logits of rows 16u + 4(l/16) + v for head l%16, summed over the
  // waves in a fixed order: wave w sums entry (u, v) = (w / 4, w % 4) of
  // every lane once, and every wave reads the sums
  if (wave < 4 || two) {  // uniform
    const int u = wave >> 2, v = wave & 3;
    float p[kAttnWaves];
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) p[w] = st.lgp[w][u][v][lane];
    st.lgf[u][v][lane] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  }
  __syncthreads();
  float lgt[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float sum = u == 0 || two ? st.lgf[u][v][lane] : 0.0f;
      lgt[u][v] = 16 * u + 4 * lg + v < nvalid ? scale * sum : -__builtin_inff();
    }
  // online softmax of head l%16 over the batch's rows (held by the lanes of
  // that head in the four lane groups)
  float mb = fmaxf(fmaxf(fmaxf(lgt[0][0], lgt[0][1]), fmaxf(lgt[0][2], lgt[0][3])),
                   fmaxf(fmaxf(lgt[1][0], lgt[1][1]), fmaxf(lgt[1][2], lgt[1][3])));
  mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
  mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
  const float m_new = fmaxf(S.m, mb);  // finite: the batch holds a row
  const float alpha = __expf(S.m - m_new);
  float ps = 0.0f, pw[8];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      pw[4 * u + v] = __expf(lgt[u][v] - m_new);
      ps += pw[4 * u + v];
    }
  ps += __shfl_xor(ps, 16, 64);
  ps += __shfl_xor(ps, 32, 64);
  S.l = S.l * alpha + ps;
  S.m = m_new;
  // rescale: accumulator element v is head 4(l/16) + v, whose factor sits
  // in lane 4(l/16) + v
  float av[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) av[v] = __shfl(alpha, 4 * lg + v, 64);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) S.acc[i][v] *= av[v];
  // acc += P V over this wave's 64 dimensions: tile t holds dimensions
  // 64w + 4n + t (n = l%16), so that a lane reads its four values of a row
  // with one LDS load.  The weights enter as two bf16 terms, hi + lo.
  const uint8_t *rb[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = 16 * (k >> 2) + 4 * lg + (k & 3);
    rb[k] = reinterpret_cast<const uint8_t *>(&raw[attn_slot(slotmap, b0, i, nvalid)][0]);
  }
  // (padding rows, i >= nvalid, read slot 0 and carry weight 0)
  auto split_weights = [&](const float (&x)[8], v8bf &hi, v8bf &lo) __attribute__((always_inline)) {
    v8s_attn h, l;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const __bf16 b = (__bf16)x[k];
      h[k] = __builtin_bit_cast(short, b);
      l[k] = bf16_bits(x[k] - (float)b);
    }
    hi = __builtin_bit_cast(v8bf, h);
    lo = __builtin_bit_cast(v8bf, l);
  };
  v8bf PH, PL;
  if (wave < kKvNope / 64) {  // E4M3 block `wave`: one power-of-two scale per row
    // the codes enter unscaled, four rows' bytes per conversion; row j's
    // weight carries 2^(s_j - E), E the running block exponent (the largest
    // scale byte of the rows met so far), and the accumulator counts in
    // units of 2^(E-127): rescaled exactly (powers of two) when E grows
    int sb[8], smax = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sb[k] = rb[k][kKvNope + 128 + wave];
      const int i = 16 * (k >> 2) + 4 * lg + (k & 3);
      smax = i < nvalid && sb[k] > smax ? sb[k] : smax;
    }
    smax = max(smax, __shfl_xor(smax, 16, 64));
    smax = max(smax, __shfl_xor(smax, 32, 64));  // every row of the batch: uniform
    if (smax > S.e) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) S.acc[i][v] = ldexpf(S.acc[i][v], S.e - smax);
      S.e = smax;
    }
    float pws[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) pws[k] = ldexpf(pw[k], sb[k] - S.e);
    split_weights(pws, PH, PL);
    uint32_t c4[8];  // E4M3 codes of dimensions 64w + 4n .. +4
#pragma unroll
    for (int k = 0; k < 8; ++k) c4[k] = *reinterpret_cast<const uint32_t *>(rb[k] + 64 * wave + 4 * lr);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // bytes t of rows k, k + 1 (twice), then of rows k .. k + 3 in order
      const uint32_t sel = (uint32_t)t | (uint32_t)(4 + t) << 8 | (uint32_t)t << 16 | (uint32_t)(4 + t) << 24;
      uint32_t q[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t x = __builtin_amdgcn_perm(c4[4 * h + 1], c4[4 * h], sel);
        const uint32_t y = __builtin_amdgcn_perm(c4[4 * h + 3], c4[4 * h + 2], sel);
        q[h] = __builtin_amdgcn_perm(y, x, 0x05040100u);
      }
      const v2bf_attn a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[0], 1.0f, false);
      const v2bf_attn a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[0], 1.0f, true);
      const v2bf_attn a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[1], 1.0f, false);
      const v2bf_attn a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[1], 1.0f, true);
      const v8bf VB = v8bf{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
      S.acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(PH, VB, S.acc[t], 0, 0, 0);
      S.acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(PL, VB, S.acc[t], 0, 0, 0);
    }
  } else {  // the RoPE values, indices 4n .. +4
    split_weights(pw, PH, PL);
    uint2 h4[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) h4[k] = *reinterpret_cast<const uint2 *>(rb[k] + kKvNope + 8 * lr);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v8s_attn vh, vl;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        short h, l;
        f16_split(((t < 2 ? h4[k].x : h4[k].y) >> (16 * (t & 1))) & 0xFFFFu, h, l);
        vh[k] = h;
        vl[k] = l;
      }
      const v8bf VH = __builtin_bit_cast(v8bf, vh), VL = __builtin_bit_cast(v8bf, vl);
      S.acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(PH, VH, S.acc[t], 0, 0, 0);
      S.acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(PL, VH, S.acc[t], 0, 0, 0);
      S.acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(PH, VL, S.acc[t], 0, 0, 0);
      S.acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(PL, VL, S.acc[t], 0, 0, 0);
    }
  }
  __syncthreads();  // the partial tiles and staged rows are reused
}

// Write the workgroup's partial: acc [head][512] and (m, l) [head][2] of
// head group g (part and ml point at the row group's partial).
__device__ __forceinline__ void attn_store(const AttnState &S, int n_heads, int g, float *__restrict__ part,
                                           float *__restrict__ ml) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  // E4M3 waves: from units of 2^(E-127) to values (exact unless the result
  // is an fp32 subnormal)
  const int ex = wave < kKvNope / 64 ? S.e - 127 : 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {  // dimensions 64w + 4 lr .. +4 of head 16g + 4 lg + v
    const int h = 16 * g + 4 * lg + v;
    if (h < n_heads)
      *reinterpret_cast<float4 *>(&part[(size_t)h * kKvDim + 64 * wave + 4 * lr]) =
          float4{ldexpf(S.acc[0][v], ex), ldexpf(S.acc[1][v], ex), ldexpf(S.acc[2][v], ex), ldexpf(S.acc[3][v], ex)};
  }
  const int hh = 16 * g + lr;
  if (wave == 0 && lg == 0 && hh < n_heads) {
    ml[2 * hh] = S.m;
    ml[2 * hh + 1] = S.l;
  }
}

// Staging of rows[0..m) (valid KV row indices, m <= kRawRows) into a stage's
// slots, in two phases so that other work runs while the rows are in flight:
// attn_stage_issue loads rows[i] (wave w takes i = w + 8u, u < 4) into
// registers, attn_stage_finish writes slot i realigned (the row's 583 bytes
// from byte 0, 146 dwords).  Lane j loads aligned dwords j, j + 64, j + 128
// of the row once; realigned dword j takes the next aligned dword from lane
// j + 1 (from lane 0's next register for j = 63).  Only dwords holding a
// byte of the row are read, so nothing past the buffer's last byte is
// touched.  The caller synchronizes before reading the slots.
constexpr int kRawDwords = (kKvRowBytes + 3) / 4;  // 146
constexpr int kStageRowsPerWave = kRawRows / kAttnWaves;
struct AttnStageRegs {
  uint32_t d[kStageRowsPerWave][3], sh[kStageRowsPerWave];
};

// indices past m re-load row m - 1 (never written): no branch around the
// loads, so they all stay in flight (m >= 1)
__device__ __forceinline__ void attn_stage_issue(const uint8_t *__restrict__ kv_rows, const int32_t *rows, int m,
                                                 AttnStageRegs &R) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kStageRowsPerWave; ++u) {
    const int i = wave + kAttnWaves * u;
    const int32_t r = __builtin_amdgcn_readfirstlane(rows[i < m ? i : m - 1]);
    const uint8_t *rb = kv_rows + (size_t)(uint32_t)r * kKvRowBytes;
    const uint32_t mis = (uint32_t)(uintptr_t)rb & 3u;
    const uint32_t *a0 = reinterpret_cast<const uint32_t *>(rb - mis);
    const int last = (int)(mis + kKvRowBytes - 1) >> 2;
    R.sh[u] = 8u * mis;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int j = lane + 64 * k;
      R.d[u][k] = a0[j < last ? j : last];
    }
  }
}

__device__ __forceinline__ void attn_stage_finish(const AttnStageRegs &R, int m, AttnRawRow *raw) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kStageRowsPerWave; ++u) {
    const int i = wave + kAttnWaves * u;
    if (i < m) {  // uniform
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int j = lane + 64 * k;
        const uint32_t up = (uint32_t)__shfl_down((int)R.d[u][k], 1, 64);
        const uint32_t wrap = (uint32_t)__shfl((int)R.d[u][k < 2 ? k + 1 : 2], 0, 64);
        const uint32_t hi = lane == 63 ? wrap : up;
        const uint32_t w = (uint32_t)(((uint64_t)hi << 32 | R.d[u][k]) >> R.sh[u]);
        if (j < kRawDwords) raw[i][j] = w;
      }
    }
  }
}

// Staging by direct-to-LDS loads, for callers that have other work to do
// while the rows are in flight and cannot hold them in registers:
// attn_stage_dma_issue copies the 148 aligned dwords that contain row rows[i]
// (i < m <= kRawRows; wave w takes i = w + 8u) into slot i as they lie in
// memory (lanes past the row's last dword re-read it, lanes past the slot
// are masked off); attn_stage_dma_finish, after the caller has waited for
// the loads (wait_vmcnt<0>) and synchronized, shifts each slot in place so
// the row starts at byte 0 (each wave reads all of a row's dwords before it
// writes any).  The caller synchronizes again before reading the slots.
__device__ __forceinline__ void attn_stage_dma_issue(const uint8_t *__restrict__ kv_rows, const int32_t *rows, int m,
                                                     AttnRawRow *raw) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kRawRows / kAttnWaves; ++u) {
    const int i = wave + kAttnWaves * u;
    if (i < m) {  // uniform
      const int32_t r = __builtin_amdgcn_readfirstlane(rows[i]);
      const uint8_t *rb = kv_rows + (size_t)(uint32_t)r * kKvRowBytes;
      const uint32_t mis = (uint32_t)(uintptr_t)rb & 3u;
      const uint8_t *a0 = uniform_ptr(rb - mis);  // scalar base, lane offsets
      const int last = (int)(mis + kKvRowBytes - 1) >> 2;  // <= 146
      const uint32_t slot = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&raw[i][0]);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int j = lane + 64 * k;
        if (j < kRawStride / 4) dma4s(a0, 4u * (uint32_t)(j < last ? j : last), slot + 256 * k);
      }
    }
  }
}

__device__ __forceinline__ void attn_stage_dma_finish(const uint8_t *__restrict__ kv_rows, const int32_t *rows, int m,
                                                      AttnRawRow *raw) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kRawRows / kAttnWaves; ++u) {
    const int i = wave + kAttnWaves * u;
    if (i < m) {  // uniform
      const int32_t r = __builtin_amdgcn_readfirstlane(rows[i]);
      const uint32_t sh = 8u * ((uint32_t)(uintptr_t)(kv_rows + (size_t)(uint32_t)r * kKvRowBytes) & 3u);
      uint32_t lo[3], hi[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int j = lane + 64 * k;
        lo[k] = raw[i][j < kRawDwords ? j : 0];
        hi[k] = raw[i][j < kRawDwords ? j + 1 : 0];
      }
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int j = lane + 64 * k;
        if (j < kRawDwords) raw[i][j] = (uint32_t)(((uint64_t)hi[k] << 32 | lo[k]) >> sh);
      }
    }
  }
}

// The merge of head h's row-group partials for dimensions d0 .. d0 + cnt
// (one per thread t < cnt): threads 0..31 form the group weights
// w_b = e^{m_b - M} (0 for empty groups), L = sum_b w_b l_b (in group order)
// and lse = M + log L into cs; then out[d] = (sum_b w_b acc_b[d]) / L, summed
// in group order (out = 0 and lse = -inf without any row).  ml, part: one
// session's partials; out_h, lse_h: head h's output row and lse (lse_h may
// be null; written by the thread of dimension 0).  All threads call it.
struct CombineShared {
  float wgt[kAttnGroups];
  float l, lse;
};

__device__ __forceinline__ void attn_combine_head(const float *ml, const float *part, int groups, int h, int d0,
                                                  int cnt, CombineShared &cs, float *out_h, float *lse_h) {
  const int t = threadIdx.x;
  const int d = d0 + (t < cnt ? t : 0);
  // every group's value of this dimension, loaded with the (m, l) pairs
  // (indices past the groups are clamped to group 0 and weigh nothing)
  float xv[kAttnGroups];
#pragma unroll
  for (int b = 0; b < kAttnGroups; ++b)
    xv[b] = part[((size_t)(b < groups ? b : 0) * CSA_MAX_HEADS + h) * kKvDim + d];
  if (t < kAttnGroups) {  // lane b holds group b's (m, l)
    const int b = t;
    const float mb = b < groups ? ml[((size_t)b * CSA_MAX_HEADS + h) * 2] : -__builtin_inff();
    const float lb = b < groups ? ml[((size_t)b * CSA_MAX_HEADS + h) * 2 + 1] : 0.0f;
    float M = mb;
#pragma unroll
    for (int o = 1; o < kAttnGroups; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, kAttnGroups));
    const float w = (M == -__builtin_inff() || mb == -__builtin_inff()) ? 0.0f : __expf(mb - M);
    cs.wgt[b] = w;
    const float wl = w * lb;
    float L = 0.0f;
    for (int c = 0; c < groups; ++c) L += __shfl(wl, c, kAttnGroups);
    if (b == 0) {
      cs.l = L;
      cs.lse = L > 0.0f ? M + logf(L) : -__builtin_inff();
    }
  }
  __syncthreads();
  if (t < cnt) {
    float X = 0.0f;
#pragma unroll
    for (int b = 0; b < kAttnGroups; ++b) {
      const float w = cs.wgt[b];
      X += w == 0.0f ? 0.0f : w * xv[b];
    }
    const float L = cs.l;
    out_h[d] = L > 0.0f ? X / L : 0.0f;
    if (lse_h && d == 0) *lse_h = cs.lse;
  }
}

// Attention over a row group's rows (in order) for head group g -> the
// partial of those heads.  Rows are staged kRawRows at a time; the next
// stage's loads are in flight while a batch is computed.  All threads call
// it.
__device__ __forceinline__ void attn_group_rows(const uint4 *qsplit, AttnStage &st, const int32_t *rows, int m,
                                                const uint8_t *__restrict__ kv_rows, float scale, int n_heads, int g,
                                                float *__restrict__ part, float *__restrict__ ml) {
  static_assert(kAttnBatch == kRawRows, "one batch per stage");
  AttnQuery q;
  load_attn_query(q, qsplit, g);
  AttnState S;
  attn_init(S);
  AttnStageRegs R;
  if (m > 0) attn_stage_issue(kv_rows, rows, m < kRawRows ? m : kRawRows, R);
  for (int b0 = 0; b0 < m; b0 += kRawRows) {
    const int cnt = m - b0 < kRawRows ? m - b0 : kRawRows;
    attn_stage_finish(R, cnt, st.raw);  // the previous batch ended with a barrier
    __syncthreads();
    const int nx = m - b0 - kRawRows;  // rows of the next stage
    if (nx > 0) attn_stage_issue(kv_rows, rows + b0 + kRawRows, nx < kRawRows ? nx : kRawRows, R);
    attn_batch(q, S, st, st.raw, nullptr, b0, cnt, scale);
  }
  attn_store(S, n_heads, g, part, ml);
}

// The same attention over m <= kRawRows rows that are already staged: the
// i-th row in order sits in slot slotmap[i]; q holds the wave's query terms
// (load_attn_query).  Same bits as attn_group_rows over those rows in that
// order.  All threads call it.
__device__ __forceinline__ void attn_staged_rows(const AttnQuery &q, AttnStage &st, const int32_t *slotmap, int m,
                                                 float scale, int n_heads, int g, float *__restrict__ part,
                                                 float *__restrict__ ml) {
  AttnState S;
  attn_init(S);
  for (int b0 = 0; b0 < m; b0 += kAttnBatch)
    attn_batch(q, S, st, st.raw, slotmap, b0, m - b0 < kAttnBatch ? m - b0 : kAttnBatch, scale);
  attn_store(S, n_heads, g, part, ml);
}

}  // namespace csa
