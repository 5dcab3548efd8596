// csa_topk_tile.hip -- fused score + per-tile heads (DS4X page, "CSA
// score/top-512 fusion": the scorer keeps exact local selections of sortable
// (score, index) keys per tile of rows, so no separate pass over a score
// array is needed to find the winners).
//
// tile_kernel (one workgroup per T-row tile of one session):
//   1. scores the tile's rows on the matrix cores (csa_score.hpp) into LDS
//      and writes them out (or reads a given score array);
//   2. finds the tile's exact top-hd keys ("heads", hd in {16, 32, 64}) and
//      writes them sorted descending to heads[tile][hd] (0-padded).
// Step 2 first bounds the hd-th key from below without sorting the tile:
// every wave finds, from the 64 per-lane maxima of its keys, a value with at
// least hd of them at or above it (a bit-by-bit search on the top 24 bits,
// one ballot per bit); the largest such bound over the waves is theta.  Only keys >= theta can be heads.  At most
// hd lanes per wave hold such keys, so there are at most 4 * hd * (T / 256)
// of them (typically 2-4 hd); they are ranked exactly against each other.
// The global selection over the heads is in csa_merge.hip.
#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "csa_score.hpp"
#include "csa_select.hpp"
#include "csa_stream.hpp"

namespace csa {

struct TileSession {
  const uint8_t *idx_rows;
  const float *scores_in;
  float *scores_out;
  int64_t n_rows;
  int hd;
};

struct TileArgs {
  TileSession s[CSA_MAX_SESSIONS];
  const uint32_t *qsplit;  // [session][kQSplitBytes / 4]
  uint64_t *heads;         // [session][heads_stride]
  int64_t heads_stride;
  int tile_rows;
};
static_assert(sizeof(TileArgs) <= 4096, "kernel argument block");

enum { kModeScore = 0, kModeScoreSelect = 1, kModeArraySelect = 2 };

constexpr int kTileThreads = 256;
constexpr int kTileWaves = kTileThreads / 64;

constexpr int kTileKPT = kMaxTileRows / kTileThreads;  // keys per thread, at most
constexpr int kRingDepth = 3;                            // chunks in flight per wave
constexpr int kTileCandCap = 256;                        // keys >= theta ranked directly

struct TileShared {
  uint8_t ring[kTileWaves][kRingDepth][kChunkSlot];  // per-wave chunk ring
  float score[kMaxTileRows];                          // scores by tile position
  uint64_t cand[kTileCandCap + 16];                   // keys >= theta (+ over-read slack)
  uint64_t theta[kTileWaves];
  uint32_t ccnt;
  SelScratch<kTileWaves> sc;
};

// Step 2: keys in registers (slot j of thread tid is tile position tid +
// 256 j, 0 = none) -> the tile's top-hd keys, sorted, at heads_out[0..hd).
__device__ void tile_heads(TileShared &sh, const uint64_t (&x)[kTileKPT], int nj, int hd,
                           uint64_t *__restrict__ heads_out) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint64_t lmax = 0;
#pragma unroll
  for (int j = 0; j < kTileKPT; ++j)
    if (j < nj) lmax = x[j] > lmax ? x[j] : lmax;
  // the largest 24-bit prefix p of the key with at least hd lane maxima at
  // or above p << 40: those hd keys are >= p << 40, a valid bound
  const uint32_t o = (uint32_t)(lmax >> 40);
  uint32_t p = 0;
#pragma unroll
  for (int b = 23; b >= 0; --b) {
    const uint32_t c = p | (1u << b);
    if (__popcll(__ballot(o >= c)) >= hd) p = c;
  }
  const uint64_t tw = (uint64_t)p << 40;
  if (lane == 0) sh.theta[wave] = tw;
  if (tid == 0) sh.ccnt = 0;
  __syncthreads();
  uint64_t theta = 1;
#pragma unroll
  for (int w = 0; w < kTileWaves; ++w) theta = sh.theta[w] > theta ? sh.theta[w] : theta;
#pragma unroll
  for (int j = 0; j < kTileKPT; ++j) {
    if (j < nj && x[j] >= theta) {
      const uint32_t p = atomicAdd(&sh.ccnt, 1u);
      if (p < kTileCandCap) sh.cand[p] = x[j];
    }
  }
  __syncthreads();
  int C = (int)sh.ccnt;
  if (C > kTileCandCap) {
    // many keys tie with or crowd above the bound: select exactly instead
    const uint64_t thr = block_kth_largest_reg<kTileWaves, kTileKPT>(x, nj, hd, theta, sh.sc);
    if (tid == 0) sh.ccnt = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTileKPT; ++j)
      if (j < nj && x[j] != 0 && x[j] >= thr) sh.cand[atomicAdd(&sh.ccnt, 1u)] = x[j];
    __syncthreads();
    C = (int)sh.ccnt;
  }
  // rank = number of larger candidates = sorted position
  for (int i = tid; i < C; i += kTileThreads) {
    const uint64_t key = sh.cand[i];
    int r = 0;
    for (int j0 = 0; j0 < C; j0 += 16) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint64_t y = sh.cand[j0 + u];
        r += (j0 + u < C && y > key) ? 1 : 0;
      }
    }
    if (r < hd) heads_out[r] = key;
  }
  for (int r = C + tid; r < hd; r += kTileThreads) heads_out[r] = 0ull;
}

// Score every row of the tile: wave w takes chunks w, w + 4, ... (64 rows
// each).  Chunks lying wholly inside the buffer stream through the wave's
// LDS ring kRingDepth - 1 chunks ahead; a final partial chunk (the buffer
// end need not be 16-byte aligned) is read with per-lane row-clamped loads.
// Each row's score goes to sh.score[position].
// Chunks of this wave that lie wholly inside the buffer.
__device__ __forceinline__ int stream_chunks(int rows, int wave) {
  const int nfull = rows / kChunkRows;  // chunks with all 64 rows present
  return nfull > wave ? (nfull - wave + kTileWaves - 1) / kTileWaves : 0;
}

// Chunk c of this wave into its ring slot (c past the last chunk reloads the
// last one: the loop keeps a fixed number of loads in flight).
__device__ __forceinline__ void stream_issue(const uint8_t *__restrict__ idx_rows, int64_t row0, int cnt, int c,
                                             TileShared &sh, int wave, int lane) {
  const int cc = c < cnt ? c : cnt - 1;
  issue_chunk(idx_rows, row0 + (int64_t)kChunkRows * (wave + kTileWaves * cc),
              (uint32_t)(uintptr_t)&sh.ring[wave][c % kRingDepth][0], lane);
}

// The first kRingDepth - 1 chunks, issued before the query fragments are
// loaded so that both latencies overlap.
__device__ __forceinline__ void stream_prologue(const uint8_t *__restrict__ idx_rows, int64_t row0, int rows,
                                                TileShared &sh, int wave, int lane) {
  const int cnt = stream_chunks(rows, wave);
  if (cnt > 0) {
#pragma unroll
    for (int c = 0; c < kRingDepth - 1; ++c) stream_issue(idx_rows, row0, cnt, c, sh, wave, lane);
  }
}

// Requires stream_prologue() and then no outstanding vector memory loads but
// those chunks.
template <int G>
__device__ __forceinline__ void score_stream(const QFrag<G> &q, const uint8_t *__restrict__ idx_rows, int64_t row0,
                                             int64_t n, int rows, TileShared &sh, int wave, int lane) {
  const int nch = (rows + kChunkRows - 1) / kChunkRows;
  const int nfull = rows / kChunkRows;  // chunks with all 64 rows present
  const int cnt = stream_chunks(rows, wave);
  // lanes 0..15 hold rows pos0 + lane of operand 0, lanes 16..31 rows
  // pos0 + lane of operand 1
  auto emit2 = [&](int pos0, const float (&s2)[2]) {
    if (lane < 32 && pos0 + lane < rows) sh.score[pos0 + lane] = score_finish(lane < 16 ? s2[0] : s2[1], 0.0f);
  };
  if (cnt > 0) {
    for (int c = 0; c < cnt; ++c) {
      stream_issue(idx_rows, row0, cnt, c + kRingDepth - 1, sh, wave, lane);
      wait_vmcnt<kChunkDma * (kRingDepth - 1)>();
      const uint8_t *base = &sh.ring[wave][c % kRingDepth][0];
      const int pos0 = kChunkRows * (wave + kTileWaves * c);
#pragma unroll
      for (int sp = 0; sp < kChunkRows / 32; ++sp) {
        RowOperand ops[2];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const uint8_t *rb = base + (32 * sp + 16 * v + (lane & 15)) * kIdxRowBytes;
          const uint32_t *w = reinterpret_cast<const uint32_t *>(rb + 16 * (lane >> 4));
          ops[v].codes = uint4{w[0], w[1], w[2], w[3]};
          ops[v].sb = rb[64 + (lane >> 4)];
        }
        float s2[2];
        score_part<G, 2>(q, ops, s2);
        emit2(pos0 + 32 * sp, s2);
      }
    }
    wait_vmcnt<0>();  // no chunk load may still be writing LDS past this point
  }
  if (nch > nfull && (nch - 1) % kTileWaves == wave) {
    const int pos0 = kChunkRows * (nch - 1);
#pragma unroll
    for (int sp = 0; sp < kChunkRows / 32; ++sp) {
      RowOperand ops[2];
#pragma unroll
      for (int v = 0; v < 2; ++v) ops[v] = load_row_operand(idx_rows, row0 + pos0 + 32 * sp + 16 * v, n, lane);
      float s2[2];
      score_part<G, 2>(q, ops, s2);
      emit2(pos0 + 32 * sp, s2);
    }
  }
}

template <int G, int MODE>
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
  const int nj = (rows + kTileThreads - 1) / kTileThreads;
  uint64_t x[kTileKPT];
  auto key_of = [&](int i, float sc) -> uint64_t {
    return ((uint64_t)score_ord(sc) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(row0 + i));
  };

  if constexpr (MODE != kModeArraySelect) {
    stream_prologue(S.idx_rows, row0, rows, sh, tid >> 6, lane);
    QFrag<G> q;
    load_qfrag<G>(q, a.qsplit + (size_t)sess * (kQSplitBytes / 4), lane, 0);
    wait_vmcnt<0>();  // query and first chunks resident: the loop's own waits count chunks only
    score_stream<G>(q, S.idx_rows, row0, n, rows, sh, tid >> 6, lane);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTileKPT; ++j) {
      const int i = tid + kTileThreads * j;
      x[j] = 0ull;
      if (j < nj && i < rows) {
        const float sc = sh.score[i];
        S.scores_out[row0 + i] = sc;
        x[j] = key_of(i, sc);
      }
    }
    if constexpr (MODE == kModeScore) return;
  } else {
    // all loads first (clamped addresses), then the keys
    float v[kTileKPT];
#pragma unroll
    for (int j = 0; j < kTileKPT; ++j) {
      const int i = tid + kTileThreads * j;
      v[j] = S.scores_in[row0 + (i < rows ? i : rows - 1)];
    }
#pragma unroll
    for (int j = 0; j < kTileKPT; ++j) {
      const int i = tid + kTileThreads * j;
      x[j] = (j < nj && i < rows) ? key_of(i, v[j]) : 0ull;
    }
  }
  tile_heads(sh, x, nj, S.hd, a.heads + (size_t)sess * a.heads_stride + (size_t)blockIdx.x * S.hd);
}

// ---------------------------------------------------------------- launcher

template <int MODE>
static hipError_t launch_tile_mode(const TileArgs &a, dim3 grid, int groups, hipStream_t st) {
  switch (groups) {
    case 1: tile_kernel<1, MODE><<<grid, kTileThreads, 0, st>>>(a); break;
    case 2: tile_kernel<2, MODE><<<grid, kTileThreads, 0, st>>>(a); break;
    case 3: tile_kernel<3, MODE><<<grid, kTileThreads, 0, st>>>(a); break;
    default: tile_kernel<4, MODE><<<grid, kTileThreads, 0, st>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_tiles(const TileJob &job, hipStream_t st) {
  TileArgs a;
  int64_t max_rows = 0;
  for (int i = 0; i < job.n_sessions; ++i) {
    a.s[i] = TileSession{job.idx_rows[i], job.scores_in[i], job.scores_out[i], job.n_rows[i], job.hd[i]};
    max_rows = job.n_rows[i] > max_rows ? job.n_rows[i] : max_rows;
  }
  if (max_rows == 0) return hipSuccess;
  a.qsplit = job.qsplit;
  a.heads = job.heads;
  a.heads_stride = job.heads_stride;
  a.tile_rows = job.tile_rows;
  const int groups = (job.n_idx_heads + 15) / 16;
  dim3 grid((unsigned)((max_rows + job.tile_rows - 1) / job.tile_rows), (unsigned)job.n_sessions);
  switch (job.mode) {
    case TileJob::kScore: return launch_tile_mode<kModeScore>(a, grid, groups, st);
    case TileJob::kScoreSelect: return launch_tile_mode<kModeScoreSelect>(a, grid, groups, st);
    default:
      tile_kernel<1, kModeArraySelect><<<grid, kTileThreads, 0, st>>>(a);
      return hipGetLastError();
  }
}

}  // namespace csa
