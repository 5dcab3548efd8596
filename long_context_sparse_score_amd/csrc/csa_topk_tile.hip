// csa_topk_tile.hip -- fused score + exact top-512 selection, without a
// full score array (DS4X page, "CSA score/top-512 fusion": per-CTA exact
// local top-512 lists of sortable (score, index) keys, then merges that keep
// float order and lower-index tie break).
//
// tile_kernel (one workgroup per T-row tile of one session):
//   1. scores the tile's rows on the matrix cores (csa_score.hpp) into LDS
//      (or reads a given score array, or only writes the scores);
//   2. selects the tile's exact top-min(512, rows) keys -> cand[tile][512]
//      (unordered, 0-padded) and its top-16 sorted descending ->
//      heads[tile][16] (0-padded).
// merge_kernel (one workgroup per session):
//   3. G = the 512th largest head over all tiles (or "everything" if there are
//      fewer).  At least 512 keys are >= G, so G lower-bounds the global
//      512th key.  A tile whose 16th head is below G holds at most 15 keys
//      >= G, all among its heads; any other ("full") tile contributes its
//      cand list.  At most 32 tiles can be full, so the candidates number at
//      most 32*512 + 512 and fit in LDS.
//   4. exact top-k_eff of the candidates, sorted -> sel_idx / sel_score.
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
};

struct TileArgs {
  TileSession s[CSA_MAX_SESSIONS];
  const uint32_t *qsplit;  // [session][kQSplitBytes / 4]
  uint64_t *cand;          // [session][cand_stride]
  uint64_t *heads;         // [session][heads_stride]
  int64_t cand_stride, heads_stride;
  int tile_rows;
};
static_assert(sizeof(TileArgs) <= 4096, "kernel argument block");

enum { kModeScore = 0, kModeScoreSelect = 1, kModeArraySelect = 2 };

constexpr int kTileThreads = 256;
constexpr int kTileWaves = kTileThreads / 64;

constexpr int kTileKPT = kMaxTileRows / kTileThreads;  // keys per thread, at most
constexpr int kRingDepth = 3;                            // chunks in flight per wave

struct TileShared {
  uint8_t ring[kTileWaves][kRingDepth][kChunkSlot];  // per-wave chunk ring
  float score[kMaxTileRows];                          // scores by tile position
  uint64_t sel[kTopK];
  uint64_t top16[16];
  uint32_t cnt, cnt16;
  SelScratch<kTileWaves> sc;
};

// Step 2 on keys held in registers (slot j of thread tid is tile position
// tid + 256 j; nj slots are live): the tile's top-512 set and sorted top-16.
__device__ void tile_select(TileShared &sh, const uint64_t (&x)[kTileKPT], int nj, int rows,
                            uint64_t *__restrict__ cand_out, uint64_t *__restrict__ heads_out) {
  const int tid = threadIdx.x;
  const int k_loc = rows < kTopK ? rows : kTopK;
  if (tid == 0) { sh.cnt = 0; sh.cnt16 = 0; }
  const uint64_t thr = block_kth_largest_reg<kTileWaves, kTileKPT>(x, nj, k_loc, 1ull, sh.sc);
#pragma unroll
  for (int j = 0; j < kTileKPT; ++j) {
    if (j < nj && x[j] != 0 && x[j] >= thr) {
      const uint32_t p = atomicAdd(&sh.cnt, 1u);
      sh.sel[p] = x[j];
      cand_out[p] = x[j];
    }
  }
  for (int p = k_loc + tid; p < kTopK; p += kTileThreads) cand_out[p] = 0ull;
  __syncthreads();
  const int kh = k_loc < 16 ? k_loc : 16;
  uint64_t y[kTopK / kTileThreads];
#pragma unroll
  for (int j = 0; j < kTopK / kTileThreads; ++j) {
    const int i = tid + kTileThreads * j;
    y[j] = i < k_loc ? sh.sel[i] : 0ull;
  }
  const uint64_t thr16 = block_kth_largest_reg<kTileWaves, kTopK / kTileThreads>(y, kTopK / kTileThreads, kh,
                                                                                  1ull, sh.sc);
#pragma unroll
  for (int j = 0; j < kTopK / kTileThreads; ++j)
    if (y[j] != 0 && y[j] >= thr16) sh.top16[atomicAdd(&sh.cnt16, 1u)] = y[j];
  __syncthreads();
  if (tid < 64) {
    const uint64_t v = wave_sort16_desc(tid < kh ? sh.top16[tid] : 0ull);
    if (tid < 16) heads_out[tid] = v;
  }
}

// Score every row of the tile: wave w takes chunks w, w + 4, ... (64 rows
// each).  Chunks lying wholly inside the buffer stream through the wave's
// LDS ring kRingDepth - 1 chunks ahead; a final partial chunk (the buffer
// end need not be 16-byte aligned) is read with per-lane row-clamped loads.
// Each row's score goes to sh.score[position].
template <int G>
__device__ __forceinline__ void score_stream(const QFrag<G> &q, const uint8_t *__restrict__ idx_rows, int64_t row0,
                                             int64_t n, int rows, TileShared &sh, int wave, int lane) {
  const int nch = (rows + kChunkRows - 1) / kChunkRows;
  const int nfull = rows / kChunkRows;  // chunks with all 64 rows present
  const int cnt = nfull > wave ? (nfull - wave + kTileWaves - 1) / kTileWaves : 0;
  auto emit2 = [&](int pos0, const float (&s2)[2]) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int pos = pos0 + 16 * v + lane;
      if (lane < 16 && pos < rows) sh.score[pos] = score_finish(s2[v], 0.0f);
    }
  };
  if (cnt > 0) {
    auto slot = [&](int k) { return (uint32_t)(uintptr_t)&sh.ring[wave][k][0]; };
    auto issue = [&](int c) {
      const int cc = c < cnt ? c : cnt - 1;
      issue_chunk(idx_rows, row0 + (int64_t)kChunkRows * (wave + kTileWaves * cc), slot(c % kRingDepth), lane);
    };
#pragma unroll
    for (int c = 0; c < kRingDepth - 1; ++c) issue(c);
    for (int c = 0; c < cnt; ++c) {
      issue(c + kRingDepth - 1);
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
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nj = (rows + kTileThreads - 1) / kTileThreads;
  uint64_t x[kTileKPT];
  auto key_of = [&](int i, uint32_t ord) -> uint64_t {
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(row0 + i));
  };

  if constexpr (MODE != kModeArraySelect) {
    QFrag<G> q;
    load_qfrag<G>(q, a.qsplit + (size_t)sess * (kQSplitBytes / 4), lane, 0);
    wait_vmcnt<0>();  // the query is resident before the chunk loads start
    score_stream<G>(q, S.idx_rows, row0, n, rows, sh, wave, lane);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTileKPT; ++j) {
      const int i = tid + kTileThreads * j;
      if (j < nj && i < rows) {
        const float sc = sh.score[i];
        if constexpr (MODE == kModeScore) S.scores_out[row0 + i] = sc;
        else x[j] = key_of(i, score_ord(sc));
      } else {
        x[j] = 0ull;
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
      x[j] = (j < nj && i < rows) ? key_of(i, score_ord(v[j])) : 0ull;
    }
  }
  tile_select(sh, x, nj, rows, a.cand + (size_t)sess * a.cand_stride + (size_t)blockIdx.x * kTopK,
              a.heads + (size_t)sess * a.heads_stride + (size_t)blockIdx.x * 16);
}

// ---------------------------------------------------------------- merge

struct MergeSession {
  const float *scores;  // score array (csa_topk) or nullptr (fused path)
  int32_t *sel_idx;
  float *sel_score;
  int64_t n_rows;
};

struct MergeArgs {
  MergeSession s[CSA_MAX_SESSIONS];
  const uint64_t *cand;
  const uint64_t *heads;
  int64_t cand_stride, heads_stride;
  int tile_rows;
  int k;
};
static_assert(sizeof(MergeArgs) <= 4096, "kernel argument block");

constexpr int kMergeThreads = 1024;
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMergeCap = 32 * kTopK + kTopK;  // candidate bound (see the file comment)
constexpr int kHeadKPT = 16;                     // heads per thread held in registers
constexpr int kMaxRegHeads = kHeadKPT * kMergeThreads;
constexpr int kCandKPT = (kMergeCap + kMergeThreads - 1) / kMergeThreads;  // 17

struct MergeShared {
  // candidate buffer of the many-tile path; the register path keeps the
  // tiles' 16th heads in it, and both reuse it for the sorted output
  uint64_t buf[kMergeCap];
  uint64_t out[kTopK];
  uint32_t full_tiles[64];
  uint32_t cnt, nfull;
  SelScratch<kMergeWaves> sc;
};
static_assert(kMaxRegHeads / 16 <= kMergeCap && kTopK <= kMergeCap, "aliases fit in buf");

__device__ void merge_write(const MergeSession &S, MergeShared &sh, int k, int k_eff) {
  const int tid = threadIdx.x;
  uint64_t *sorted = sh.buf;
  if (k_eff > 0) block_rank_sort_desc<kMergeThreads>(sh.out, k_eff, sorted);
  for (int t = tid; t < k; t += kMergeThreads) {
    if (t < k_eff) {
      const uint64_t x = sorted[t];
      const uint32_t row = key_row(x);
      S.sel_idx[t] = (int32_t)row;
      if (S.sel_score) S.sel_score[t] = S.scores ? S.scores[row] : key_score(x);
    } else {
      S.sel_idx[t] = -1;
      if (S.sel_score) S.sel_score[t] = -__builtin_inff();
    }
  }
}

__global__ void __launch_bounds__(kMergeThreads) merge_kernel(const MergeArgs a) {
  const int sess = blockIdx.x;
  const MergeSession &S = a.s[sess];
  const int64_t n = S.n_rows;
  const int k = a.k;
  const int k_eff = (int)(n < k ? n : k);
  const int tid = threadIdx.x;
  __shared__ MergeShared sh;
  if (k_eff == 0) {
    merge_write(S, sh, k, 0);
    return;
  }
  const int64_t nt = (n + a.tile_rows - 1) / a.tile_rows;
  const uint64_t *heads = a.heads + (size_t)sess * a.heads_stride;
  const uint64_t *cand = a.cand + (size_t)sess * a.cand_stride;
  const int nh = (int)(nt * 16);
  if (tid == 0) { sh.cnt = 0; sh.nfull = 0; }

  if (nh <= kMaxRegHeads) {
    uint64_t *tile16 = sh.buf;
    // heads in registers: slot j of thread tid is head tid + 1024 j
    const int nj = (nh + kMergeThreads - 1) / kMergeThreads;
    uint64_t h[kHeadKPT];
#pragma unroll
    for (int j = 0; j < kHeadKPT; ++j) {
      const int i = tid + kMergeThreads * j;
      h[j] = heads[i < nh ? i : nh - 1];
    }
#pragma unroll
    for (int j = 0; j < kHeadKPT; ++j) {
      const int i = tid + kMergeThreads * j;
      if (i >= nh) h[j] = 0ull;
      else if ((i & 15) == 15) tile16[i >> 4] = h[j];
    }
    // 3. G: the 512th largest head (1 if there are fewer)
    const uint64_t G = block_kth_largest_reg<kMergeWaves, kHeadKPT>(h, nj, kTopK, 1ull, sh.sc);
    // candidates: heads >= G of tiles that are not full, in registers ...
#pragma unroll
    for (int j = 0; j < kHeadKPT; ++j) {
      const int i = tid + kMergeThreads * j;
      if (!(h[j] != 0 && h[j] >= G && tile16[i >> 4] < G)) h[j] = 0ull;
    }
    // ... and the cand lists of full tiles (at most 32 + 1 of them)
    for (int64_t t = tid; t < nt; t += kMergeThreads)
      if (tile16[t] >= G) sh.full_tiles[atomicAdd(&sh.nfull, 1u)] = (uint32_t)t;
    __syncthreads();
    const int ncand = (int)sh.nfull * kTopK;
    uint64_t c[kCandKPT];
#pragma unroll
    for (int j = 0; j < kCandKPT; ++j) {
      const int i = tid + kMergeThreads * j;
      const int ii = i < ncand ? i : 0;
      c[j] = ncand ? cand[(size_t)sh.full_tiles[ii / kTopK] * kTopK + (ii % kTopK)] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < kCandKPT; ++j) {
      const int i = tid + kMergeThreads * j;
      if (!(i < ncand && c[j] >= G)) c[j] = 0ull;
    }
    // 4. exact top-k_eff of the candidates (heads and cand slots together)
    uint64_t u[kHeadKPT + kCandKPT];
#pragma unroll
    for (int j = 0; j < kHeadKPT; ++j) u[j] = h[j];
#pragma unroll
    for (int j = 0; j < kCandKPT; ++j) u[kHeadKPT + j] = c[j];
    const uint64_t thr =
        block_kth_largest_reg<kMergeWaves, kHeadKPT + kCandKPT>(u, kHeadKPT + kCandKPT, k_eff, G, sh.sc);
    if (tid == 0) sh.cnt = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kHeadKPT + kCandKPT; ++j)
      if (u[j] != 0 && u[j] >= thr) sh.out[atomicAdd(&sh.cnt, 1u)] = u[j];
    __syncthreads();
  } else {
    // Many tiles: the same steps, reading the heads from memory each pass.
    const uint64_t G =
        block_kth_largest<kMergeWaves>([&](int i) { return heads[i]; }, nh, kTopK, 1ull, sh.sc);
    for (int i = tid; i < nh; i += kMergeThreads) {
      const uint64_t x = heads[i];
      if (x >= G && heads[(i | 15)] < G) sh.buf[atomicAdd(&sh.cnt, 1u)] = x;
    }
    for (int64_t t = tid; t < nt; t += kMergeThreads)
      if (heads[t * 16 + 15] >= G) sh.full_tiles[atomicAdd(&sh.nfull, 1u)] = (uint32_t)t;
    __syncthreads();
    const int nfull = (int)sh.nfull;
    for (int i = tid; i < nfull * kTopK; i += kMergeThreads) {
      const uint64_t x = cand[(size_t)sh.full_tiles[i / kTopK] * kTopK + (i % kTopK)];
      if (x >= G) sh.buf[atomicAdd(&sh.cnt, 1u)] = x;
    }
    __syncthreads();
    const int nc = (int)sh.cnt;
    const uint64_t thr = block_kth_largest<kMergeWaves>([&](int i) { return sh.buf[i]; }, nc, k_eff, G, sh.sc);
    if (tid == 0) sh.cnt = 0;
    __syncthreads();
    for (int i = tid; i < nc; i += kMergeThreads) {
      const uint64_t x = sh.buf[i];
      if (x >= thr) sh.out[atomicAdd(&sh.cnt, 1u)] = x;
    }
    __syncthreads();
  }
  merge_write(S, sh, k, k_eff);
}

// ---------------------------------------------------------------- launchers

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
    a.s[i] = TileSession{job.idx_rows[i], job.scores_in[i], job.scores_out[i], job.n_rows[i]};
    max_rows = job.n_rows[i] > max_rows ? job.n_rows[i] : max_rows;
  }
  if (max_rows == 0) return hipSuccess;
  a.qsplit = job.qsplit;
  a.cand = job.cand;
  a.heads = job.heads;
  a.cand_stride = job.cand_stride;
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

hipError_t launch_merge(const TileJob &job, int32_t *const *sel_idx, float *const *sel_score, int k,
                        hipStream_t st) {
  MergeArgs a;
  for (int i = 0; i < job.n_sessions; ++i)
    a.s[i] = MergeSession{job.mode == TileJob::kArraySelect ? job.scores_in[i] : nullptr, sel_idx[i], sel_score[i],
                          job.n_rows[i]};
  a.cand = job.cand;
  a.heads = job.heads;
  a.cand_stride = job.cand_stride;
  a.heads_stride = job.heads_stride;
  a.tile_rows = job.tile_rows;
  a.k = k;
  merge_kernel<<<job.n_sessions, kMergeThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa
