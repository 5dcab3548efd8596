// csa_topk_tile.hip -- fused score + per-tile heads (DS4X page, "CSA
// score/top-512 fusion": the scorer keeps exact local selections of sortable
// (score, index) keys per tile of rows, so no separate pass over a score
// array is needed to find the winners).
//
// tile_kernel (one workgroup per T-row tile of one session):
//   1. scores the tile's rows on the matrix cores (csa_score.hpp) into LDS
//      and writes them out (or reads a given score array);
//   2. finds the tile's exact top-hd keys ("heads", hd in {8, 16, 32, 64}) and
//      writes them sorted descending to heads[tile][hd] (0-padded).
// Step 2 first bounds the hd-th key from below without sorting the tile:
// every wave splits its 64 lanes into hd groups and takes the smallest group
// maximum of the lanes' largest keys (score part), a value with at least hd
// keys at or above it; the largest such bound over the waves is theta.  Only
// keys >= theta can be heads: typically a few times hd of them, ranked
// exactly against each other (an exact k-th selection replaces theta when
// they overflow the candidate buffer).
// The global selection over the heads is in csa_merge.hip.
#include "csa_attn.hpp"
#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "csa_score.hpp"
#include "csa_select.hpp"
#include "csa_stream.hpp"

namespace csa {

struct TileSession {
  const uint8_t *idx_rows;
  float *scores;        // written (scoring modes) or read (array mode)
  const float *q, *w;   // indexer query and head weights
  const float *q_attn;  // attention query
  int64_t n_rows;
  int hd;
};

struct TileArgs {
  TileSession s[CSA_MAX_SESSIONS];
  uint4 *attn_q;  // attention query split [session][kAttnQVecs], or null
  uint64_t *heads;  // [session][heads_stride]
  int64_t heads_stride;
  int tile_rows;
  int n_idx_heads, n_attn_heads;
  int write_heads;  // scoring launches: also find and write the tile heads
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
    float score[kMaxTileRows];  // scores by tile position
  } a;
};
static_assert(sizeof(TileShared) <= 80 * 1024, "two workgroups per compute unit");

// Step 2: the tile's scores in sh.a.score[0..rows) and, per thread, the
// largest score part (score_ord) over its positions tid + 256 j -> the
// tile's top-hd keys, sorted, at heads_out[0..hd).
__device__ __forceinline__ void tile_heads(TileShared &sh, uint32_t o, int rows, int64_t row0, int hd,
                                           uint64_t *__restrict__ heads_out) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  auto key_at = [&](int i) __attribute__((always_inline)) {
    return make_key(sh.a.score[i], (uint32_t)(row0 + i));
  };
  // the largest 24-bit prefix p with at least hd lane maxima at or above
  // p << 8 (two bits per step): those hd keys are >= p << 40
  const uint32_t o24 = o >> 8;
  uint32_t p = 0;
#pragma unroll
  for (int b = 22; b >= 0; b -= 2) {
    const uint32_t c1 = p | (1u << b), c2 = p | (2u << b), c3 = p | (3u << b);
    const int n1 = __popcll(__ballot(o24 >= c1));
    const int n2 = __popcll(__ballot(o24 >= c2));
    const int n3 = __popcll(__ballot(o24 >= c3));
    p = n3 >= hd ? c3 : (n2 >= hd ? c2 : (n1 >= hd ? c1 : p));
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
    // (exactly hd keys are >= the hd-th largest)
    const uint64_t thr = block_kth_largest<kTileWaves>(key_at, rows, hd, theta, sh.h.sc);
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
    if (r < hd) heads_out[r] = key;
  }
  for (int r = C + tid; r < hd; r += kTileThreads) heads_out[r] = 0ull;
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

// Score the tile's rows into sh.a.score[0..rows) (and out[0..rows)).
// Wave w owns chunks w, w + 4, w + 8, ... of the tile (64 rows each) and
// scores them for every head group, so each row is read from LDS once and
// the group parts of a row meet in the lane that holds it; the waves run
// without workgroup barriers.  A chunk wholly inside the buffer comes in
// direct-to-LDS, kRingDepth - 1 chunks ahead, into the wave's own ring; a
// chunk cut by the buffer end is copied with clamped per-lane loads.
// Query terms: wave g brings the fp32 query of head group g (16 heads,
// 8 KB) and all the weights direct-to-LDS into its ring slots 1 and 2 ahead
// of its first chunk, so they arrive first and the split runs while the
// chunk is in flight.  Each head's 512 bytes land at a 528-byte stride, so
// the split's reads spread over the LDS banks; each wave then writes its
// group's terms over its own staging area (16-byte quad j of lane l at
// 16 (64 j + l)), and after one barrier every wave reads every group's
// terms.  The chunks after the first are issued once a second barrier has
// released the slots.
template <int G>
__device__ __forceinline__ uint32_t score_tile(const float *__restrict__ qh, const float *__restrict__ wh,
                                               int n_idx_heads, const uint8_t *__restrict__ idx_rows, int64_t row0,
                                               int64_t n, int rows, float *__restrict__ out, TileShared &sh) {
  static_assert(G == 1 || G == 2 || G == 4, "head groups per workgroup");
  static_assert(kRingDepth >= 3, "the query is staged in ring slots 1 and 2");
  constexpr int kStageHead = 528, kStageW = 16 * kStageHead;
  static_assert(kStageW + 256 <= 2 * kChunkBytes, "group query + weights fit two ring slots");
  static_assert(kXchQuads * 64 * 16 <= kStageW, "the terms leave the weights alone");
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
  uint8_t *const stage = &sh.ring[wave][1][0];
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
  if (direct(0))
    wait_vmcnt<kChunkDma>();
  else
    wait_vmcnt<0>();
  QFrag<1> q[G];
  {
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
      split_qfrag(mine, x);
      // the terms over the staging area (this wave's reads of it come first):
      // the lane's 32 words (6 per term, then the packed scales) as eight
      // 16-byte quads, quad j of lane l at stage + 16 (64 j + l)
      uint32_t w[kXchQuads * 4];
#pragma unroll
      for (int t = 0; t < kTerms; ++t)
#pragma unroll
        for (int i = 0; i < 6; ++i) w[6 * t + i] = (uint32_t)mine.a[0][t][i];
#pragma unroll
      for (int j = 0; j < kScaleWords; ++j) w[6 * kTerms + j] = (uint32_t)mine.scw[0][j];
#pragma unroll
      for (int j = 6 * kTerms + kScaleWords; j < kXchQuads * 4; ++j) w[j] = 0u;
      uint4 *x16 = reinterpret_cast<uint4 *>(stage) + lane;
#pragma unroll
      for (int j = 0; j < kXchQuads; ++j) x16[64 * j] = uint4{w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 *x16 = reinterpret_cast<const uint4 *>(&sh.ring[g][1][0]) + lane;
      uint32_t w[kXchQuads * 4];
#pragma unroll
      for (int j = 0; j < kXchQuads; ++j) {
        const uint4 v = x16[64 * j];
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
    // the weights (in slot 2, which the exchange leaves alone)
    const float *wl = reinterpret_cast<const float *>(stage + kStageW);
#pragma unroll
    for (int g = 0; g < G; ++g) load_qweights(q[g], wl, n_idx_heads, g, lane);
    __syncthreads();  // every wave has read the terms and weights: the slots are free
#pragma unroll
    for (int t = 1; t <= kRingDepth - 2; ++t)
      if (t < nmy) fill(t);
  }

  uint32_t omax = 0;  // largest score part of this thread's rows
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
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    v4f c[4][1], cn[4][1];
    group_dots<4>(q[0], ops, c);
#pragma unroll
    for (int g = 1; g < G; ++g) {
      group_dots<4>(q[g], ops, cn);
      group_acc4(q[g - 1], c, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) c[r][0] = cn[r][0];
    }
    group_acc4(q[G - 1], c, acc);
    // lane l: row l of the chunk, summed over every head
    float v = rows_reduce4(acc);
    const int p = kChunkRows * chunk(s) + lane;
    if (p < rows) {
      v = score_finish(v, 0.0f);
      sh.a.score[p] = v;
      out[p] = v;
      const uint32_t so = score_ord(v);
      omax = so > omax ? so : omax;
    }
  }
  __syncthreads();
  return omax;
}

// ARRAY: the scores are given (csa_topk).  The scoring launches of csa_score
// and of the decode step run the same code (the heads are a runtime choice),
// so both produce the same bits: the scaled matrix-core accumulation may
// round differently under a different instruction schedule.
template <int G, bool ARRAY>
__global__ void __launch_bounds__(kTileThreads, 2) tile_kernel(const TileArgs a) {
  const int sess = blockIdx.y;
  const TileSession &S = a.s[sess];
  const int64_t n = S.n_rows;
  const int T = a.tile_rows;
  const int64_t row0 = (int64_t)blockIdx.x * T;
  if (row0 >= n) return;
  const int rows = (int)((n - row0) < T ? (n - row0) : T);
  __shared__ TileShared sh;
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t o = 0;  // largest score part of this thread's positions
  if constexpr (!ARRAY) {
    uint4 *const aq = a.attn_q ? a.attn_q + (size_t)sess * kAttnQVecs : nullptr;
    const float *const qa = S.q_attn;
    const int n_attn_heads = a.n_attn_heads;
    auto attn_split = [=]() __attribute__((always_inline)) {
      if (aq) {
        // this workgroup's share of the session's attention query split
        // (read by the selection kernel that follows), spread over the
        // first half of the tiles: they are dispatched first and finish
        // while the second half still scores, so the split stays off the
        // kernel's tail
        const int nt = (int)((n + T - 1) / T);
        const int nw = nt > 1 ? nt / 2 : 1;
        const int per = (kAttnQTasks + nw - 1) / nw;
        const int b = (int)blockIdx.x;
        const int t1 = (b + 1) * per < kAttnQTasks ? (b + 1) * per : kAttnQTasks;
        if (b < nw)
          for (int t = b * per + tid; t < t1; t += kTileThreads) attn_q_split_task(qa, n_attn_heads, aq, t);
      }
    };
    o = score_tile<G>(S.q, S.w, a.n_idx_heads, S.idx_rows, row0, n, rows, S.scores + row0, sh);
    attn_split();
    if (!a.write_heads) return;
  } else {
    // the given scores into LDS, four loads in flight per thread
    const float *src = S.scores + row0;
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
          const uint32_t so = score_ord(v[u]);
          o = so > o ? so : o;
        }
      }
    }
    __syncthreads();
  }
  tile_heads(sh, o, rows, row0, S.hd, a.heads + (size_t)sess * a.heads_stride + (size_t)blockIdx.x * S.hd);
}

// ---------------------------------------------------------------- launcher

static hipError_t launch_scoring(const TileArgs &a, dim3 grid, int groups, hipStream_t st) {
  // three groups run as four: the query split holds zero terms and weights
  // for heads past n_idx_heads, which add exact zeros
  switch (groups) {
    case 1: tile_kernel<1, false><<<grid, kTileThreads, 0, st>>>(a); break;
    case 2: tile_kernel<2, false><<<grid, kTileThreads, 0, st>>>(a); break;
    default: tile_kernel<4, false><<<grid, kTileThreads, 0, st>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_tiles(const TileJob &job, hipStream_t st) {
  TileArgs a;
  int64_t max_rows = 0;
  for (int i = 0; i < job.n_sessions; ++i) {
    float *scores = job.mode == TileJob::kArraySelect ? const_cast<float *>(job.scores_in[i]) : job.scores_out[i];
    a.s[i] = TileSession{job.idx_rows[i], scores, job.q[i], job.w[i], job.q_attn[i], job.n_rows[i], job.hd[i]};
    max_rows = job.n_rows[i] > max_rows ? job.n_rows[i] : max_rows;
  }
  if (max_rows == 0) return hipSuccess;
  a.attn_q = job.mode == TileJob::kScoreSelect ? job.attn_q : nullptr;
  a.n_idx_heads = job.n_idx_heads;
  a.n_attn_heads = job.n_attn_heads;
  a.heads = job.heads;
  a.heads_stride = job.heads_stride;
  a.tile_rows = job.tile_rows;
  const int groups = (job.n_idx_heads + 15) / 16;
  dim3 grid((unsigned)((max_rows + job.tile_rows - 1) / job.tile_rows), (unsigned)job.n_sessions);
  switch (job.mode) {
    case TileJob::kScore:
      a.write_heads = 0;
      return launch_scoring(a, grid, groups, st);
    case TileJob::kScoreSelect:
      a.write_heads = 1;
      return launch_scoring(a, grid, groups, st);
    default:
      a.write_heads = 1;
      tile_kernel<1, true><<<grid, kTileThreads, 0, st>>>(a);
      return hipGetLastError();
  }
}

}  // namespace csa
