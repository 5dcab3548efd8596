// csa_topk_tile.hip -- fused filter score + per-tile heads (DS4X page, "CSA
// score/top-512 fusion": the scorer keeps exact local selections of sortable
// (score, index) keys per tile of rows, so no pass over a full score array is
// needed to find the winners).
//
// tile_kernel (one workgroup per T-row tile of one session):
//   1. scores the tile's rows with the matrix-core filter (csa_score.hpp)
//      and brackets each row's exact score, l_j <= S_j <= u_j (csa_bound.hpp),
//      into LDS; the brackets' constants come from the query split of the
//      same workgroup (with a given score array, csa_topk: l = u = S);
//   2. finds the tile's top-(hd+1) keys by upper bound, key = (u_j, row j)
//      (larger u first, lower row on ties; hd in {8, 16, 32, 64}), and writes
//      the first hd ("heads", rank-major: rank r of tile t at r * nt + t, so
//      the best heads of all tiles come first) with their lower-bound keys
//      (l_j, row j), and the (hd+1)-th ("next": every other row of the tile
//      has a key at or below it).  A row's bracket is kept as u (fp32) and
//      beta rounded up to bf16; the heads' lower bounds are rebuilt from them
//      (row_lower; exactly l = u when beta = 0, as for given scores).
// Nothing is written per row: the refine kernel (csa_refine.hip) takes the
// heads that can reach the top-k and, for the rare tile whose "next" can,
// every row of it, and scores them exactly.
// Step 2 first bounds the (hd+1)-th key from below without sorting the tile:
// every wave splits its 64 lanes into groups and takes the smallest group
// maximum of the lanes' largest keys (score part), a value with at least
// hd+1 keys at or above it; the largest such bound over the waves is theta.
// Only keys >= theta can be among the top hd+1: typically a few times hd of
// them, ranked exactly against each other (an exact k-th selection replaces
// theta when they overflow the candidate buffer).
#include <hip/hip_ext.h>

#include "csa_attn.hpp"
#include "csa_bound.hpp"
#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "csa_score.hpp"
#include "csa_select.hpp"
#include "csa_stream.hpp"

namespace csa {

struct TileSession {
  const uint8_t *idx_rows;
  const float *scores_in;  // array mode: the given scores
  const float *q, *w;      // indexer query and head weights
  int64_t n_rows;
  int hd;
};

struct TileArgs {
  TileSession s[CSA_MAX_SESSIONS];
  uint64_t *hkey;    // [session][heads_stride]: head keys by upper bound, rank-major [hd][nt]
  uint64_t *hlow;    // [session][heads_stride]: the heads' lower-bound keys, same order
  uint64_t *hnext;   // [session][tiles_stride]: per tile its (hd+1)-th key, 0 if none
  float *bnd_up, *bnd_lo;  // bounds mode: the brackets of every row (one session)
  float *qhat;             // quantized query: [session][64][128] fp32 copy for the rescoring, or null
  int64_t heads_stride, tiles_stride;
  int tile_rows;
  int n_idx_heads;
  int mode;  // TileJob::Mode
  int shared_rows;  // > 0: every session scores the same rows; the grid is
                    // one-dimensional, tile-major (the sessions of a tile run
                    // side by side and share its rows in the L2)
};
static_assert(sizeof(TileArgs) <= 4096, "kernel argument block");


// Two 4-wave workgroups per compute unit.
constexpr int kTileThreads = 256;
constexpr int kTileWaves = kTileThreads / 64;

constexpr int kRingDepth = 4;     // chunks resident per wave: D - 1 in flight
constexpr int kTileCandCap = 256; // keys >= theta ranked directly
constexpr int kXchWords = kTerms * 6 + kScaleWords;  // fp6 term registers + packed scales per lane
constexpr int kXchQuads = (kXchWords + 3) / 4;       // ... exchanged as 16-byte quads
static_assert(kRingDepth >= 2 && kRingDepth <= 4, "ring depth");
static_assert(kChunkBytes % 16 == 0, "direct-to-LDS pieces stay aligned");

struct TileShared {
  union {
    alignas(16) uint8_t ring[kTileWaves][kRingDepth][kChunkBytes];  // one ring per wave (step 1)
    struct {
      uint64_t cand[kTileCandCap + 16];  // keys >= theta (+ over-read slack)
      uint64_t theta[kTileWaves];
      uint32_t ccnt;
      SelScratch<kTileWaves> sc;
    } h;  // step 2: the ring is drained by then
  };
  struct {
    union {
      float score[kMaxTileRows];  // upper bounds u by tile position (from the streaming loop on)
      struct {
        double zpart[kMaxGroups][4];  // bound constants per head group and block
        uint4 xq[kMaxGroups][64];     // the last quad of each group's exchanged terms
      } pro;                          // prologue only
    };
    uint16_t beta[kMaxTileRows];    // the bracket half-widths, bf16 rounded up
  } a;
};
static_assert(sizeof(TileShared) <= 80 * 1024, "two workgroups per compute unit");

// x >= 0 (or +inf) rounded up to bf16 bits.
__device__ __forceinline__ uint16_t bf16_round_up(float x) {
  const uint32_t b = __float_as_uint(x);
  return (uint16_t)((b >> 16) + ((b & 0xFFFFu) != 0u ? 1u : 0u));
}

// The lower bound of a row from its upper bound u and bf16 half-width bits:
// u lies at most 6 ulp(u) above s~ + beta (csa_bound.hpp), so
// l = rounddown(u - 2 beta - 8 ulp(u)) <= s~ - beta; l = u when beta = 0
// (given scores, exact).
__device__ __forceinline__ float row_lower(float u, uint16_t bb) {
  const float beta = __uint_as_float((uint32_t)bb << 16);
  if (beta == 0.0f) return u;  // exact (given scores)
  if (!(fabsf(u) <= 3.40282347e38f) || !(beta <= 3.40282347e38f)) return -__builtin_inff();
  const double ulp = (double)f32_next_up(fabsf(u)) - (double)fabsf(u);
  return f32_round_down((double)u - 2.0 * (double)beta - 8.0 * ulp);
}

// Step 2: the tile's upper bounds in sh.a.score[0..rows) (half-widths in
// sh.a.beta) and, per thread, the largest score part (score_ord) over its
// positions tid + 256 j -> the tile's top-(hd+1) keys by upper bound: rank r
// < hd to hkey_out[r * rstride] with its lower-bound key to
// hlow_out[r * rstride], the (hd+1)-th to *next_out (0 if the tile has at
// most hd rows; heads past the rows are 0).
__device__ __forceinline__ void tile_heads(TileShared &sh, uint32_t o, int rows, int64_t row0, int hd,
                                           uint64_t *__restrict__ hkey_out, uint64_t *__restrict__ hlow_out,
                                           int64_t rstride, uint64_t *__restrict__ next_out) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int want = hd + 1;  // heads and next
  auto key_at = [&](int i) __attribute__((always_inline)) {
    return make_key(sh.a.score[i], (uint32_t)(row0 + i));
  };
  // the largest 24-bit prefix p with at least `want` lane maxima at or above
  // p << 8 (two bits per step): those keys are >= p << 40
  const uint32_t o24 = o >> 8;
  uint32_t p = 0;
#pragma unroll
  for (int b = 22; b >= 0; b -= 2) {
    const uint32_t c1 = p | (1u << b), c2 = p | (2u << b), c3 = p | (3u << b);
    const int n1 = __popcll(__ballot(o24 >= c1));
    const int n2 = __popcll(__ballot(o24 >= c2));
    const int n3 = __popcll(__ballot(o24 >= c3));
    p = n3 >= want ? c3 : (n2 >= want ? c2 : (n1 >= want ? c1 : p));
  }
  if (lane == 0) sh.h.theta[wave] = (uint64_t)p << 40;
  if (tid == 0) sh.h.ccnt = 0;
  __syncthreads();
  uint64_t theta = 1;  // also excludes empty positions
#pragma unroll
  for (int w = 0; w < kTileWaves; ++w) theta = sh.h.theta[w] > theta ? sh.h.theta[w] : theta;
  // keys >= lb, eight positions per thread at a time (their loads issued
  // together), one LDS atomic per wave and batch: the wave's keys take
  // consecutive positions.  A wave whose largest score parts are all below
  // the bound's holds no candidate and skips the scan.
  const int nj = (rows + kTileThreads - 1) / kTileThreads;
  auto gather = [&](uint64_t lb, uint32_t cap) __attribute__((always_inline)) {
    if (__ballot(o >= (uint32_t)(lb >> 32)) == 0) return;
    for (int j0 = 0; j0 < nj; j0 += 8) {
      bool ok[8];
      uint64_t kx[8], m[8];
      float sv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = tid + kTileThreads * (j0 + u);
        sv[u] = sh.a.score[i < rows ? i : 0];
      }
      uint32_t tot = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = tid + kTileThreads * (j0 + u);
        kx[u] = make_key(sv[u], (uint32_t)(row0 + i));
        ok[u] = i < rows && kx[u] >= lb;
        m[u] = __ballot(ok[u]);
        tot += (uint32_t)__popcll(m[u]);
      }
      if (tot != 0) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&sh.h.ccnt, tot);
        base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t q = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m[u] >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m[u], 0u));
          if (ok[u] && q < cap) sh.h.cand[q] = kx[u];
          base += (uint32_t)__popcll(m[u]);
        }
      }
    }
  };
  gather(theta, (uint32_t)kTileCandCap);
  __syncthreads();
  int C = (int)sh.h.ccnt;
  if (C > kTileCandCap) {
    // many keys tie with or crowd above the bound: select exactly instead
    // (exactly `want` keys are >= the want-th largest)
    const uint64_t thr = block_kth_largest<kTileWaves>(key_at, rows, want, theta, sh.h.sc);
    if (tid == 0) sh.h.ccnt = 0;
    __syncthreads();
    gather(thr, (uint32_t)kTileCandCap);
    __syncthreads();
    C = (int)sh.h.ccnt;
  }
  // rank = number of larger candidates = sorted position
  for (int i = tid; i < C; i += kTileThreads) {
    const uint64_t key = sh.h.cand[i];
    int r = 0;
    for (int j0 = 0; j0 < C; j0 += 16) {
      uint64_t y[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) y[u] = sh.h.cand[j0 + u];  // the slack covers j0 + u >= C
#pragma unroll
      for (int u = 0; u < 16; ++u) r += (j0 + u < C && y[u] > key) ? 1 : 0;
    }
    if (r < hd) {
      const uint32_t i = key_row(key) - (uint32_t)row0;
      hkey_out[r * rstride] = key;
      hlow_out[r * rstride] = make_key(row_lower(sh.a.score[i], sh.a.beta[i]), key_row(key));
    } else if (r == hd) {
      *next_out = key;
    }
  }
  for (int r = C + tid; r < hd; r += kTileThreads) {
    hkey_out[r * rstride] = 0ull;
    hlow_out[r * rstride] = 0ull;
  }
  if (C <= hd && tid == 0) *next_out = 0ull;
}

// Sums of fp64 values over lanes on the DPP network (the 32-bit halves move
// separately; lanes without a source add +0).  row_sum_f64: inclusive scan
// within each 16-lane row (lane 15 of a row ends with its sum);
// wave_sum_f64: the whole wave's sum in every lane.  Summation order is
// immaterial to the callers (bound constants with a rounding margin).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double row_sum_f64(double v) {
  v += dpp_f64<0x111, 0xF>(v);  // row_shr:1
  v += dpp_f64<0x112, 0xF>(v);  // row_shr:2
  v += dpp_f64<0x114, 0xF>(v);  // row_shr:4
  v += dpp_f64<0x118, 0xF>(v);  // row_shr:8
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = row_sum_f64(v);
  v += dpp_f64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Rows [r0, r0 + 64) of a chunk that ends past the buffer: lane l copies
// row min(r0 + l, n - 1) to dst + 68 l with ordinary loads (the compiler
// waits for them before the LDS stores; rows past n are scored and dropped).
__device__ __forceinline__ void copy_chunk_clamped(const uint8_t *__restrict__ rows, int64_t r0, int64_t n,
                                                   uint8_t *dst, int lane) {
  int64_t r = r0 + lane;
  r = r < n ? r : n - 1;
  const uint32_t *src = reinterpret_cast<const uint32_t *>(rows + r * kIdxRowBytes);
  uint32_t v[kIdxRowBytes / 4];
#pragma unroll
  for (int i = 0; i < kIdxRowBytes / 4; ++i) v[i] = src[i];
  uint32_t *d = reinterpret_cast<uint32_t *>(dst + lane * kIdxRowBytes);
#pragma unroll
  for (int i = 0; i < kIdxRowBytes / 4; ++i) d[i] = v[i];
}

// Wait until this wave's chunk of the current step is in LDS, `later` being
// the number of later steps whose chunk this wave has already issued
// direct-to-LDS.  Vector loads complete in order, so at most
// later * kChunkDma outstanding loads means the current chunk is done; a
// score store still outstanding only lengthens the wait.
__device__ __forceinline__ void wait_chunk(int later) {
  if (kRingDepth > 3 && later >= 2)
    wait_vmcnt<2 * kChunkDma>();
  else if (kRingDepth > 2 && later >= 1)
    wait_vmcnt<kChunkDma>();
  else
    wait_vmcnt<0>();
}

// This lane's operands of the chunk at `base` in LDS: operand i is rows
// 16 i .. + 16, the lane taking row l%16's code bytes [16(l/16), +16) and
// scale byte l/16.
__device__ __forceinline__ void load_ops(const uint8_t *base, RowOperand (&ops)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t *rb = base + (16 * i + (lane & 15)) * kIdxRowBytes;
    const uint32_t *w = reinterpret_cast<const uint32_t *>(rb + 16 * (lane >> 4));
    ops[i].codes = uint4{w[0], w[1], w[2], w[3]};
    ops[i].sb = rb[64 + (lane >> 4)];
  }
}

// Score the tile's rows and bracket their exact scores: u into
// sh.a.score[0..rows), the half-width into sh.a.beta (and, in the bounds
// mode, u and l to bnd_up / bnd_lo).
// Wave w owns chunks w, w + 4, w + 8, ... of the tile (64 rows each) and
// scores them for every head group, so each row is read from LDS once and
// the group parts of a row meet in the lane that holds it; the waves run
// without workgroup barriers.  A chunk wholly inside the buffer comes in
// direct-to-LDS, kRingDepth - 1 chunks ahead, into the wave's own ring; a
// chunk cut by the buffer end is copied with clamped per-lane loads.
// Query terms: wave g brings the fp32 query of head group g (16 heads,
// 8 KB) and all the weights direct-to-LDS into its ring slots 2 and 3 ahead
// of its first two chunks (slots 0 and 1), so they arrive first and the
// split runs while the chunks are in flight.  Each head's 512 bytes land at
// a 528-byte stride, so the split's reads spread over the LDS banks.  Once
// the wave holds its query values, slot 2 is free and the wave issues its
// third chunk there (a wave without a query group issues it with the first
// two).  Each wave then writes its group's terms as 16-byte quads (quad
// j < 4 of lane l at 16 (64 j + l) in its slot 3, below the weights; the
// last quad in LDS outside the ring) and its part of the bound constants;
// after one barrier every wave reads every group's terms and the constants,
// and after a second the loop may refill slot 3 (the loop issues the rest,
// always in order).
template <int G, int QF>
__device__ __forceinline__ uint32_t score_tile(const float *__restrict__ qh, const float *__restrict__ wh,
                                               int n_idx_heads, const uint8_t *__restrict__ idx_rows, int64_t row0,
                                               int64_t n, int rows, TileShared &sh, float *__restrict__ bnd_up,
                                               float *__restrict__ bnd_lo, float *__restrict__ qhat) {
  static_assert(G == 1 || G == 2 || G == 4, "head groups per workgroup");
  static_assert(kRingDepth == 4, "the query is staged in ring slots 2 and 3, chunks 0 and 1 go ahead");
  constexpr int kStageHead = 528, kStageW = 16 * kStageHead;
  static_assert(kStageW + 256 <= 2 * kChunkBytes, "group query + weights fit two ring slots");
  static_assert(kXchQuads == 5 && 4 * 64 * 16 == kStageW - kChunkBytes, "four quads in slot 3 below the weights, one outside");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: chunk bookkeeping stays scalar
  const int nch = (rows + kChunkRows - 1) / kChunkRows;
  const int nfc = rows / kChunkRows;  // chunks wholly inside the buffer
  const int nmy = wave < nch ? (nch - wave + kTileWaves - 1) / kTileWaves : 0;  // this wave's chunks
  auto chunk = [&](int s) __attribute__((always_inline)) { return wave + kTileWaves * s; };
  // this wave's first chunk (uniform) and the lanes' piece offsets
  const uint8_t *const wave_rows = uniform_ptr(idx_rows + (row0 + (int64_t)kChunkRows * wave) * kIdxRowBytes);
  const ChunkLanes cl = chunk_lanes(lane);
  auto fill = [&](int s) __attribute__((always_inline)) {
    const int c = chunk(s);
    uint8_t *dst = &sh.ring[wave][s % kRingDepth][0];
    if (c < nfc)
      issue_chunk_s(wave_rows + (size_t)s * (kTileWaves * kChunkBytes), cl, (uint32_t)(uintptr_t)dst, lane);
    else if (c < nch)
      copy_chunk_clamped(idx_rows, row0 + (int64_t)kChunkRows * c, n, dst, lane);
  };
  auto direct = [&](int s) __attribute__((always_inline)) { return s < nmy && chunk(s) < nfc; };

  // staging: head 16 wave + j (clamped to the last one) at stage + 528 j,
  // one 512-byte load per head (the 16-byte pad spreads the split's reads
  // over the banks), the weights at stage + kStageW
  uint8_t *const stage = &sh.ring[wave][2][0];
  const uint32_t stage_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)stage);
  if (wave < G && lane < 32) {
    // the head rows' addresses are uniform: scalar bases, one lane offset
    const uint32_t voff = 16u * (uint32_t)lane;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int h = 16 * wave + j < n_idx_heads ? 16 * wave + j : n_idx_heads - 1;
      dma16s(reinterpret_cast<const uint8_t *>(qh + (size_t)h * 128), voff, stage_lds + kStageHead * j);
    }
  }
  dma4(wh + (lane < n_idx_heads ? lane : n_idx_heads - 1), stage_lds + kStageW);
  if (nmy > 0) fill(0);
  if (nmy > 1) fill(1);
  const bool early2 = wave >= G;  // uniform: no query staged in slot 2
  if (early2 && nmy > 2) fill(2);
  // the query and weights have landed once at most the chunks issued after
  // them are outstanding (loads complete in issue order; direct chunks are
  // a prefix of the wave's chunks, and a clamped copy waits for itself)
  switch ((direct(0) ? 1 : 0) + (direct(1) ? 1 : 0) + (early2 && direct(2) ? 1 : 0)) {
    case 3: wait_vmcnt<3 * kChunkDma>(); break;
    case 2: wait_vmcnt<2 * kChunkDma>(); break;
    case 1: wait_vmcnt<kChunkDma>(); break;
    default: wait_vmcnt<0>(); break;
  }
  QFrag<1> q[G];
  FilterBoundF F;
  {
    FilterBound B;
    const float *wl = reinterpret_cast<const float *>(stage + kStageW);  // this wave's copy of the weights
    if (wave < G) {
      float x[32];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 v =
            *reinterpret_cast<const float4 *>(stage + kStageHead * (lane & 15) + 128 * (lane >> 4) + 16 * i);
        x[4 * i] = v.x;
        x[4 * i + 1] = v.y;
        x[4 * i + 2] = v.z;
        x[4 * i + 3] = v.w;
      }
      QFrag<1> mine;
      QFragNorms nm;
      if constexpr (QF == kQueryMxfp4) {
        float deq[32];
        nm = quantize_qfrag_fp4(mine, x, deq);
        // one workgroup of the session keeps the quantized query (fp32) for
        // the exact rescoring
        const int hq = 16 * wave + (lane & 15);
        if (qhat && hq < n_idx_heads) {
          float4 *dst = reinterpret_cast<float4 *>(qhat + (size_t)hq * 128 + 32 * (lane >> 4));
#pragma unroll
          for (int i = 0; i < 8; ++i) dst[i] = float4{deq[4 * i], deq[4 * i + 1], deq[4 * i + 2], deq[4 * i + 3]};
        }
      } else {
        nm = split_qfrag(mine, x);
      }
      // the query values are in registers: slot 2 takes the third chunk
      wait_lgkmcnt0();
      if (nmy > 2) fill(2);
      // this lane's part of the bound constants: |w_h| (rho + 2^-15 A) for its
      // (head, block) fragment, summed over the group's 16 heads per block
      // (lanes 16 b .. 16 b + 15 hold block b); fp64 so that no range is lost
      const int h = 16 * wave + (lane & 15);
      const double wa = h < n_idx_heads ? fabs((double)wl[h]) : 0.0;
      double cz = wa == 0.0 ? 0.0 : wa * ((double)nm.rho + 0x1p-15 * nm.mag);
      cz = row_sum_f64(cz);  // lane 15 of each 16-lane row: the row's sum
      if ((lane & 15) == 15) sh.a.pro.zpart[wave][lane >> 4] = cz;
      // the terms (this wave's reads of its staged query come first): the
      // lane's words (6 per term, then the packed scales) as 16-byte quads
      uint32_t w[kXchQuads * 4];
#pragma unroll
      for (int t = 0; t < kTerms; ++t)
#pragma unroll
        for (int i = 0; i < 6; ++i) w[6 * t + i] = (uint32_t)mine.a[0][t][i];
#pragma unroll
      for (int j = 0; j < kScaleWords; ++j) w[6 * kTerms + j] = (uint32_t)mine.scw[0][j];
#pragma unroll
      for (int j = 6 * kTerms + kScaleWords; j < kXchQuads * 4; ++j) w[j] = 0u;
      uint4 *x16 = reinterpret_cast<uint4 *>(&sh.ring[wave][3][0]) + lane;
#pragma unroll
      for (int j = 0; j < 4; ++j) x16[64 * j] = uint4{w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
      sh.a.pro.xq[wave][lane] = uint4{w[16], w[17], w[18], w[19]};
    }
    // Z_abs from the weights (every wave, its own copy): 2^-117 sum_h |w_h|
    double wsum = lane < n_idx_heads ? fabs((double)wl[lane]) : 0.0;
    wsum = wave_sum_f64(wsum);
    __syncthreads();
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      double z = 0.0;
#pragma unroll
      for (int g = 0; g < G; ++g) z += sh.a.pro.zpart[g][b];
      B.z[b] = z * (6.0 * (1.0 + 0x1p-10));
    }
    B.zabs = wsum * 0x1p-117;
    F = bound_f32(B);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 *x16 = reinterpret_cast<const uint4 *>(&sh.ring[g][3][0]) + lane;
      uint32_t w[kXchQuads * 4];
#pragma unroll
      for (int j = 0; j < kXchQuads; ++j) {
        const uint4 v = j < 4 ? x16[64 * j] : sh.a.pro.xq[g][lane];
        w[4 * j] = v.x;
        w[4 * j + 1] = v.y;
        w[4 * j + 2] = v.z;
        w[4 * j + 3] = v.w;
      }
#pragma unroll
      for (int t = 0; t < kTerms; ++t)
        q[g].a[0][t] = v8i{(int)w[6 * t], (int)w[6 * t + 1], (int)w[6 * t + 2], (int)w[6 * t + 3],
                           (int)w[6 * t + 4], (int)w[6 * t + 5], 0, 0};
#pragma unroll
      for (int j = 0; j < kScaleWords; ++j) q[g].scw[0][j] = (int)w[6 * kTerms + j];
    }
    // the weights (in slot 3, which the exchange leaves alone)
#pragma unroll
    for (int g = 0; g < G; ++g) load_qweights(q[g], wl, n_idx_heads, g, lane);
    __syncthreads();  // every wave has read the terms and weights: slot 3 is free
  }

  uint32_t omax = 0;  // largest score part of this thread's upper bounds
  // With the fp32 query (three products per group and row block) a chunk's
  // last group of products, its partial sums over the other groups, its
  // scale bytes and this lane's tile position are carried into the next
  // step: the last group's epilogue, the row sums and the bracket run behind
  // the next chunk's first products (the same arithmetic in the same order).
  // The MXFP4 query (one product) finishes each chunk in its own step.
  constexpr bool kCarry = QF == kQueryFp32;
  float accp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  v4f cp[4][1];
  uint32_t sbp = 0;
  int pp = 0;
  auto finish = [&]() __attribute__((always_inline)) {
    group_acc4(q[G - 1], cp, accp);
    // lane l: row l of the chunk, summed over every head (the sign of a zero
    // is immaterial to the bracket), and its bracket from the row's four
    // scale bytes
    const float v = rows_reduce4(accp);
    if (pp < rows) {
      float up, lo;
      float beta;
      if (bnd_up) {  // uniform (the bounds mode)
        beta = row_bracket<true>(v, sbp, F, up, lo);
        bnd_up[pp] = up;
        bnd_lo[pp] = lo;
      } else {
        beta = row_bracket<false>(v, sbp, F, up, lo);
      }
      sh.a.score[pp] = up;
      sh.a.beta[pp] = bf16_round_up(beta);
      const uint32_t so = score_ord(up);
      omax = so > omax ? so : omax;
    }
  };
  for (int s = 0; s < nmy; ++s) {
    int later = 0;
#pragma unroll
    for (int t = 1; t <= kRingDepth - 2; ++t) later += direct(s + t) ? 1 : 0;
    wait_chunk(later);
    // the slot refilled next held chunk s - 1, whose LDS reads completed
    // before its products were formed
    if (s + kRingDepth - 1 < nmy) fill(s + kRingDepth - 1);
    // every row of the chunk is scored, also past the tile's rows in a last
    // partial chunk (stale LDS bytes; those scores are dropped); the products
    // of the next group are issued before the current group's epilogue
    const uint8_t *base = &sh.ring[wave][s % kRingDepth][0];
    RowOperand ops[4];
    load_ops(base, ops);
    const uint32_t sb = *reinterpret_cast<const uint32_t *>(base + kIdxRowBytes * lane + 64);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    v4f c[4][1], cn[4][1];
    group_dots<4, QF>(q[0], ops, c);
    if constexpr (kCarry) {
      if (s > 0) finish();  // the previous chunk
    }
#pragma unroll
    for (int g = 1; g < G; ++g) {
      group_dots<4, QF>(q[g], ops, cn);
      group_acc4(q[g - 1], c, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) c[r][0] = cn[r][0];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      cp[r][0] = c[r][0];
      accp[r] = acc[r];
    }
    sbp = sb;
    pp = kChunkRows * chunk(s) + lane;
    if constexpr (!kCarry) finish();
  }
  if constexpr (kCarry) {
    if (nmy > 0) finish();
  }
  __syncthreads();
  return omax;
}

// Modes (TileJob::Mode): kFilter scores the rows (the decode step), kArray
// takes given scores as exact (csa_topk: l = u = the score), kBounds scores
// and writes every row's bracket (a test entry point; no heads).
template <int G, bool ARRAY, int QF>
__global__ void __launch_bounds__(kTileThreads, 2) tile_kernel(const TileArgs a) {
  const int sess = a.shared_rows ? (int)(blockIdx.x % (unsigned)a.shared_rows) : (int)blockIdx.y;
  const int tile = a.shared_rows ? (int)(blockIdx.x / (unsigned)a.shared_rows) : (int)blockIdx.x;
  const TileSession &S = a.s[sess];
  const int64_t n = S.n_rows;
  const int T = a.tile_rows;
  const int64_t row0 = (int64_t)tile * T;
  if (row0 >= n) return;
  const int rows = (int)((n - row0) < T ? (n - row0) : T);
  __shared__ TileShared sh;
  const int tid = threadIdx.x;
  uint32_t o = 0;  // largest score part of this thread's positions
  if constexpr (!ARRAY) {
    const bool bounds = a.mode == TileJob::kBounds;
    float *qhat = (QF == kQueryMxfp4 && a.qhat && tile == 0) ? a.qhat + (size_t)sess * CSA_MAX_HEADS * 128 : nullptr;
    o = score_tile<G, QF>(S.q, S.w, a.n_idx_heads, S.idx_rows, row0, n, rows, sh, bounds ? a.bnd_up + row0 : nullptr,
                          bounds ? a.bnd_lo + row0 : nullptr, qhat);
    if (bounds) return;
  } else {
    // the given scores into LDS (exact: both bounds), four loads in flight
    // per thread
    const float *src = S.scores_in + row0;
    for (int j0 = 0; j0 < rows; j0 += 4 * kTileThreads) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = j0 + kTileThreads * u + tid;
        v[u] = src[i < rows ? i : rows - 1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = j0 + kTileThreads * u + tid;
        if (i < rows) {
          sh.a.score[i] = v[u];
          sh.a.beta[i] = 0;
          const uint32_t so = score_ord(v[u]);
          o = so > o ? so : o;
        }
      }
    }
    __syncthreads();
  }
  // rank-major heads of the session: rank r of tile t at r * nt + t
  const int64_t nt = (n + T - 1) / T;
  const size_t hb = (size_t)sess * a.heads_stride + (size_t)tile;
  tile_heads(sh, o, rows, row0, S.hd, a.hkey + hb, a.hlow + hb, nt,
             a.hnext + (size_t)sess * a.tiles_stride + tile);
}

// ---------------------------------------------------------------- launcher

template <int G, int QF>
static void launch_scoring_g(const TileArgs &a, dim3 grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  if (e0)
    hipExtLaunchKernelGGL(tile_kernel<G, false, QF>, grid, dim3(kTileThreads), 0, st, e0, e1, 0, a);
  else
    tile_kernel<G, false, QF><<<grid, kTileThreads, 0, st>>>(a);
}

template <int QF>
static void launch_scoring_q(const TileArgs &a, dim3 grid, int groups, hipStream_t st, hipEvent_t e0,
                             hipEvent_t e1) {
  // three groups run as four: the query split holds zero terms and weights
  // for heads past n_idx_heads, which add exact zeros
  switch (groups) {
    case 1: launch_scoring_g<1, QF>(a, grid, st, e0, e1); break;
    case 2: launch_scoring_g<2, QF>(a, grid, st, e0, e1); break;
    default: launch_scoring_g<4, QF>(a, grid, st, e0, e1); break;
  }
}

static hipError_t launch_scoring(const TileArgs &a, dim3 grid, int groups, int qfmt, hipStream_t st,
                                 hipEvent_t e0, hipEvent_t e1) {
  if (qfmt == kQueryMxfp4)
    launch_scoring_q<kQueryMxfp4>(a, grid, groups, st, e0, e1);
  else
    launch_scoring_q<kQueryFp32>(a, grid, groups, st, e0, e1);
  return hipGetLastError();
}

hipError_t launch_tiles(const TileJob &job, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_end) {
  TileArgs a;
  int64_t max_rows = 0;
  for (int i = 0; i < job.n_sessions; ++i) {
    a.s[i] = TileSession{job.idx_rows[i], job.scores_in[i], job.q[i], job.w[i], job.n_rows[i], job.hd[i]};
    max_rows = job.n_rows[i] > max_rows ? job.n_rows[i] : max_rows;
  }
  if (max_rows == 0) {  // nothing to score: the events mark the empty stage
    hipError_t e = ev_start ? hipEventRecord(ev_start, st) : hipSuccess;
    if (e == hipSuccess && ev_end) e = hipEventRecord(ev_end, st);
    return e;
  }
  a.n_idx_heads = job.n_idx_heads;
  a.hkey = job.hkey;
  a.hlow = job.hlow;
  a.hnext = job.hnext;
  a.bnd_up = job.bnd_up;
  a.bnd_lo = job.bnd_lo;
  a.qhat = job.qhat;
  a.heads_stride = job.heads_stride;
  a.tiles_stride = job.tiles_stride;
  a.tile_rows = job.tile_rows;
  a.mode = (int)job.mode;
  // sessions over the same rows (multi-token scoring): a tile-major grid
  bool shared = job.n_sessions > 1;
  for (int i = 1; i < job.n_sessions; ++i)
    shared = shared && job.idx_rows[i] == job.idx_rows[0] && job.n_rows[i] == job.n_rows[0];
  a.shared_rows = shared ? job.n_sessions : 0;
  const int groups = (job.n_idx_heads + 15) / 16;
  const unsigned nt = (unsigned)((max_rows + job.tile_rows - 1) / job.tile_rows);
  dim3 grid = shared ? dim3(nt * (unsigned)job.n_sessions, 1u) : dim3(nt, (unsigned)job.n_sessions);
  if (job.mode == TileJob::kArray) {
    if (ev_start)
      hipExtLaunchKernelGGL(tile_kernel<1, true, kQueryFp32>, grid, dim3(kTileThreads), 0, st, ev_start, ev_end, 0, a);
    else
      tile_kernel<1, true, kQueryFp32><<<grid, kTileThreads, 0, st>>>(a);
    return hipGetLastError();
  }
  return launch_scoring(a, grid, groups, job.query_format, st, ev_start, ev_end);
}

}  // namespace csa
