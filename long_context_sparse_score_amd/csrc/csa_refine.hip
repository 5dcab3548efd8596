// csa_refine.hip -- exact scores of the rows that can still reach the top-k
// (DS4X page, "CSA score/top-512 fusion": the fused selection keeps the same
// float score order and lower-index tie break as a separate exact top-k).
//
// The score the selection orders by is the lightning-indexer score
//     S_j = fl32( sum_h w_h * max(0, sum_i q_hi * k_ji) ),
// evaluated in fp64 with i ascending inside each head and h ascending
// outside (each product q_hi * k_ji of an fp32 query value and a decoded
// fp32 row value is exact in fp64, so fma(q, k, d) = d + q * k; w_h *
// max(0, d_h) is rounded, then added), rounded once to fp32, -0 stored as
// +0.  Every row this kernel scores gets exactly that value.
//
// Inputs: per tile of the score kernel its hd heads (keys by upper bound
// u_j, with lower-bound keys (l_j, row j)), rank-major (the best head of
// every tile, then the second, ...), and its "next" key (the largest key of
// its other rows).  Every workgroup of a session derives the same
//   G = a lower bound on the k_eff-th largest lower-bound key over the first
//       kRefBoundHeads heads (block_bound): at least k_eff rows have an exact
//       key >= G, so the k_eff-th largest exact key is >= G (the best heads
//       of all tiles hold nearly all of the top-k, so G stays close to it);
//   full tiles = tiles whose next key is >= G: one of their other rows may
//       reach the top-k, so every row of such a tile is scored;
//   candidates = heads with key >= G outside full tiles.
// A row outside both sets has an exact key at or below its upper-bound key,
// which is below G, so it is not in the top-k.
// Items (per session): the head slots (nh of them, in the heads' rank-major
// order: a candidate's exact key, 0 = "no key" otherwise), followed by the
// rows of the full tiles in tile order.  The selection kernel takes the top-k of the
// items' keys.  Wave w of the launch's nw waves (per session) takes items w,
// w + nw, ..., so the candidates spread over the whole chip.
// Other modes: given scores (csa_topk: the key of the given score) and every
// row (csa_score: the exact score of each row, written as fp32).
// In the decode step the workgroups also split the attention query (its
// three bf16 terms in the matrix-core operand order of csa_attn.hpp), a
// share each, for the selection kernel that follows.
#include "csa_attn.hpp"
#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "csa_select.hpp"

namespace csa {

constexpr int kRefThreads = 512;
constexpr int kRefWaves = kRefThreads / 64;
static_assert(kRefWaves == kRefineWaves, "the host's view of the workgroup");
constexpr int kRefKPT = 2;                             // bound heads per thread in registers
constexpr int kRefBoundHeads = kRefThreads * kRefKPT;  // 1024: the heads G is taken over
constexpr int kQStride = 132;  // floats per query head in LDS: rows 528 B apart spread the lanes over banks
constexpr int kRefMaxFull = 4096;  // full tiles listed per session (beyond: every row is an item)

struct RefineSession {
  const uint8_t *idx_rows;
  const float *q, *w;  // indexer query [H][128] and head weights
  float *scores;       // csa_topk: the given scores (read); csa_score: the output
  const float *q_attn;  // decode step: the attention query [n_attn_heads][512]
  int64_t n_rows;
  int hd;
};

struct RefineArgs {
  RefineSession s[CSA_MAX_SESSIONS];
  const uint64_t *hkey;  // [session][heads_stride]: rank-major head keys (upper bounds)
  const uint64_t *hlow;  // [session][heads_stride]: their lower-bound keys
  const uint64_t *hnext;  // [session][tiles_stride]
  uint64_t *items;       // [session][items_stride]
  uint32_t *count;       // [session]: number of items
  uint4 *attn_q;         // decode step: the attention query split [session][kAttnQVecs], or null
  int64_t heads_stride, tiles_stride, items_stride;
  int tile_rows;
  int n_idx_heads, n_attn_heads;
  int k;
  int mode;  // RefineJob::Mode
};
static_assert(sizeof(RefineArgs) <= 4096, "kernel argument block");

struct RefineShared {
  float q[CSA_MAX_HEADS][kQStride];  // the fp32 indexer query
  float w[CSA_MAX_HEADS];
  double kv[kRefWaves][2][128];  // per wave: the decoded rows being scored (exact fp32 values, as fp64)
  double pv[kRefWaves][2][64];   // per wave: their heads' terms w_h max(0, d_h)
  BoundShared<kRefWaves> bs;
  uint32_t full_tile[kRefMaxFull];
  uint32_t wcnt[kRefWaves];
  uint32_t nfull;
  int all_rows;  // more full tiles than listed: every row is an item
};

// Wave-level ordering of LDS traffic between lanes (LDS accesses of one wave
// complete in issue order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lane l's bytes of a row: code byte l (values 2l, 2l + 1) and the scale byte
// of its block.
struct RowBytes {
  uint32_t code, scale;
};
__device__ __forceinline__ RowBytes load_row_bytes(const uint8_t *__restrict__ idx_rows, int64_t row) {
  const int lane = threadIdx.x & 63;
  const uint8_t *r = idx_rows + (size_t)row * kIdxRowBytes;
  return RowBytes{r[lane], r[64 + (lane >> 4)]};
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ int64_t readlane_i64(int64_t x, int l) { return (int64_t)readlane_u64((uint64_t)x, l); }
__device__ __forceinline__ double readlane_f64(double x, int l) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// The exact scores S of N <= 2 rows (see the file comment) from their bytes,
// computed by one wave: lane l decodes row values 2l and 2l + 1 exactly as
// fp32 (an E2M1 value times 2^(e-127): exact, or +-inf on overflow, NaN for
// a 0xFF scale) and stores them as fp64 in LDS; lane h forms d_h in fp64
// over i ascending from its fp32 query row in LDS and the row values (one
// read serves every lane), the rows' chains interleaved and each step's
// operands read a step ahead so the reads overlap the arithmetic.  The
// heads' terms w_h max(0, d_h) (exactly +0 for lanes past n_heads) go to LDS
// and every lane adds them in head order, sixteen reads at a time, up to
// n_heads rounded up to 16: a +0 term leaves the sum unchanged (the sum
// starts at +0 and cannot become -0), so this is the reference's sum over
// the n_heads heads.
// out[r] is S of row r in every lane.
template <int N>
__device__ __forceinline__ void exact_scores(const RowBytes (&rb)[N], int n_heads, RefineShared &sh, float (&out)[N]) {
  static_assert(N == 1 || N == 2, "rows per call");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < N; ++r) {
    const float sc = ue8m0_scale(rb[r].scale);
    const float k0 = e2m1_value(rb[r].code & 15u) * sc, k1 = e2m1_value(rb[r].code >> 4) * sc;
    *reinterpret_cast<double2 *>(&sh.kv[wave][r][2 * lane]) = double2{(double)k0, (double)k1};
  }
  wave_lds_sync();
  const bool head = lane < n_heads;
  const float *qh = &sh.q[head ? lane : 0][0];
  double d[N];
  float4 qn = *reinterpret_cast<const float4 *>(qh);
  double2 kn0[N], kn1[N];
#pragma unroll
  for (int r = 0; r < N; ++r) {
    d[r] = 0.0;
    kn0[r] = *reinterpret_cast<const double2 *>(&sh.kv[wave][r][0]);
    kn1[r] = *reinterpret_cast<const double2 *>(&sh.kv[wave][r][2]);
  }
#pragma unroll 4
  for (int i = 0; i < 128; i += 4) {
    const float4 qc = qn;
    double2 kc0[N], kc1[N];
#pragma unroll
    for (int r = 0; r < N; ++r) {
      kc0[r] = kn0[r];
      kc1[r] = kn1[r];
    }
    const int in = i + 4 < 128 ? i + 4 : i;  // the last step re-reads its own operands
    qn = *reinterpret_cast<const float4 *>(qh + in);
#pragma unroll
    for (int r = 0; r < N; ++r) {
      kn0[r] = *reinterpret_cast<const double2 *>(&sh.kv[wave][r][in]);
      kn1[r] = *reinterpret_cast<const double2 *>(&sh.kv[wave][r][in + 2]);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of this step's arithmetic
    const double q0 = qc.x, q1 = qc.y, q2 = qc.z, q3 = qc.w;
#pragma unroll
    for (int r = 0; r < N; ++r) {
      d[r] = __builtin_fma(q0, kc0[r].x, d[r]);
      d[r] = __builtin_fma(q1, kc0[r].y, d[r]);
      d[r] = __builtin_fma(q2, kc1[r].x, d[r]);
      d[r] = __builtin_fma(q3, kc1[r].y, d[r]);
    }
  }
  const double wh = (double)sh.w[head ? lane : 0];
#pragma unroll
  for (int r = 0; r < N; ++r) sh.pv[wave][r][lane] = head ? wh * (d[r] > 0.0 ? d[r] : 0.0) : 0.0;
  wave_lds_sync();
  double acc[N];
#pragma unroll
  for (int r = 0; r < N; ++r) acc[r] = 0.0;
#pragma unroll 1
  for (int c = 0; c < n_heads; c += 16) {  // (the +0 terms past n_heads are skipped)
    double2 v[N][8];
#pragma unroll
    for (int r = 0; r < N; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[r][j] = *reinterpret_cast<const double2 *>(&sh.pv[wave][r][c + 2 * j]);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < N; ++r) acc[r] = (acc[r] + v[r][j].x) + v[r][j].y;
  }
#pragma unroll
  for (int r = 0; r < N; ++r) {
    const float f = (float)acc[r];
    out[r] = f == 0.0f ? 0.0f : f;
  }
  wave_lds_sync();  // kv and pv are reused by the wave's next rows
}
__device__ __forceinline__ float exact_score(const RowBytes &rb, int n_heads, RefineShared &sh) {
  const RowBytes r1[1] = {rb};
  float f[1];
  exact_scores<1>(r1, n_heads, sh, f);
  return f[0];
}

// The fp32 indexer query (padded rows) and weights into LDS, all loads in
// flight together (no barrier here).
__device__ __forceinline__ void load_query(const float *__restrict__ q, const float *__restrict__ w, int H,
                                           RefineShared &sh) {
  const int tid = threadIdx.x;
  constexpr int kQPer = CSA_MAX_HEADS * 32 / kRefThreads;  // float4 per thread
  // every load is issued (heads past H read the last head, in this
  // workgroup's own lines) and its value zeroed after: no branch, so no
  // early wait for loads issued before
  float4 qv[kQPer];
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int t = tid + kRefThreads * u, h = t >> 5, c = t & 31;
    qv[u] = reinterpret_cast<const float4 *>(q + (size_t)(h < H ? h : H - 1) * 128)[c];
  }
  const float wl = w[tid < H ? tid : H - 1];
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int t = tid + kRefThreads * u;
    *reinterpret_cast<float4 *>(&sh.q[t >> 5][4 * (t & 31)]) = (t >> 5) < H ? qv[u] : float4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  if (tid < CSA_MAX_HEADS) sh.w[tid] = tid < H ? wl : 0.0f;
}

// Rows whose bytes each wave prefetches at the start, before the bound is
// known (the rows of its first two head items' keys), so that the usual one
// or two candidates per wave need no load after the bound.
constexpr int kRefPrefetch = 2;

template <bool EXACT>  // EXACT: rows scored exactly (decode step, csa_score); else given scores (csa_topk)
__global__ void __launch_bounds__(kRefThreads) refine_kernel(const RefineArgs a) {
  const int sess = blockIdx.y;
  const RefineSession &S = a.s[sess];
  const int64_t n = S.n_rows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int H = a.n_idx_heads;
  constexpr bool exact = EXACT;
  __shared__ RefineShared sh;
  const uint32_t nw = gridDim.x * kRefWaves;               // waves per session
  const uint32_t gw = blockIdx.x * kRefWaves + (uint32_t)wave;  // this wave

  if (EXACT && (a.mode == RefineJob::kAll || a.mode == RefineJob::kKeysAll)) {
    // every row: its exact score (csa_score) or its exact key as an item (a
    // short history's decode step: the filter would cost more than it
    // saves), rows gw + 2 nw t and gw + 2 nw t + nw scored as a pair
    const bool keys = a.mode == RefineJob::kKeysAll;
    uint64_t *items = a.items + (size_t)sess * a.items_stride;
    if (keys && blockIdx.x == 0 && tid == 0) a.count[sess] = (uint32_t)n;
    load_query(S.q, S.w, H, sh);
    lds_sync();
    for (int64_t r0 = gw; r0 < n; r0 += 2 * (int64_t)nw) {
      const int64_t r1 = r0 + nw;
      const RowBytes b0 = load_row_bytes(S.idx_rows, r0);
      const RowBytes b1 = load_row_bytes(S.idx_rows, r1 < n ? r1 : r0);
      float f[2];
      if (r1 < n) {
        const RowBytes rbs[2] = {b0, b1};
        exact_scores<2>(rbs, H, sh, f);
      } else {
        f[0] = exact_score(b0, H, sh);
        f[1] = 0.0f;
      }
      if (lane == 0) {
        if (keys) {
          items[r0] = make_key(f[0], (uint32_t)r0);
          if (r1 < n) items[r1] = make_key(f[1], (uint32_t)r1);
        } else {
          S.scores[r0] = f[0];
          if (r1 < n) S.scores[r1] = f[1];
        }
      }
    }
    if (keys && a.attn_q) {  // this workgroup's share of the attention query split
      const int per = (kAttnQTasks + (int)gridDim.x - 1) / (int)gridDim.x;
      const int t1 = ((int)blockIdx.x + 1) * per < kAttnQTasks ? ((int)blockIdx.x + 1) * per : kAttnQTasks;
      for (int t = (int)blockIdx.x * per + tid; t < t1; t += kRefThreads)
        attn_q_split_task(S.q_attn, a.n_attn_heads, a.attn_q + (size_t)sess * kAttnQVecs, t);
    }
    return;
  }

  const int T = a.tile_rows, hd = S.hd;
  const int k_eff = (int)(n < a.k ? n : a.k);
  const int64_t nt = (n + T - 1) / T;
  const int64_t nh = nt * hd;
  const uint64_t *hkey = a.hkey + (size_t)sess * a.heads_stride;
  const uint64_t *hlow = a.hlow + (size_t)sess * a.heads_stride;
  const uint64_t *hnext = a.hnext + (size_t)sess * a.tiles_stride;
  uint64_t *items = a.items + (size_t)sess * a.items_stride;
  if (k_eff == 0) {
    if (blockIdx.x == 0 && tid == 0) a.count[sess] = 0;
    return;
  }
  if (tid == 0) { sh.nfull = 0; sh.all_rows = 0; }

  // Loads, issued in the order their results are needed: this wave's first
  // head items' keys and the bound's lower-bound keys, the query, the
  // attention query values of this workgroup's first split tasks, then the
  // head items' row bytes; everything after is synchronised through LDS only
  // (lds_sync), so these stay in flight across the bound's barriers.
  // (lane u: head item gw + nw u, the first of this wave's rounds)
  // (a lane past the heads reads its wave's first head: no line is read by
  // every wave)
  // The values are masked where they are used, not here: a select right
  // after a load would wait for it before the next loads are issued.
  const int64_t i_first = gw + (int64_t)nw * lane;
  const uint64_t xk_raw = hkey[i_first < nh ? i_first : (gw < nh ? gw : nh - 1)];
  // G over the lower-bound keys of the first heads (a prefix of the
  // rank-major order: every tile's best heads), two per thread
  // the first 512 tiles' next keys (the full-tile test after the bound)
  const uint64_t nx_first = hnext[tid < nt ? tid : nt - 1];
  const int64_t nb = nh < kRefBoundHeads ? nh : kRefBoundHeads;
  uint64_t lk_raw[kRefKPT];
#pragma unroll
  for (int j = 0; j < kRefKPT; ++j) {
    const int64_t i = tid + (int64_t)kRefThreads * j;
    lk_raw[j] = hlow[i < nb ? i : nb - 1];
  }
  if constexpr (EXACT) load_query(S.q, S.w, H, sh);
  // this workgroup's share of the attention query split (decode step):
  // threads past the share read its first task (no branch around the loads)
  const int qper = (kAttnQTasks + (int)gridDim.x - 1) / (int)gridDim.x;
  const int qt0 = (int)blockIdx.x * qper;
  const int qt1 = qt0 + qper < kAttnQTasks ? qt0 + qper : kAttnQTasks;
  float qx[8];
  if (a.attn_q) attn_q_load(S.q_attn, a.n_attn_heads, qt0 + tid < qt1 ? qt0 + tid : qt0, qx);
  // the rows of lanes 0 and 1's keys (speculatively: candidates or not)
  const uint64_t xk = i_first < nh ? xk_raw : 0ull;
  RowBytes pb[kRefPrefetch] = {};
  if constexpr (EXACT) {
    const int64_t fallback = (int64_t)(gw % (uint64_t)n);  // a row of its own for a wave without keys
#pragma unroll
    for (int u = 0; u < kRefPrefetch; ++u) {
      const uint64_t x = readlane_u64(xk, u);
      pb[u] = load_row_bytes(S.idx_rows, x != 0 ? (int64_t)key_row(x) : fallback);
    }
  }

  // 1. the bound G
  uint64_t lk[kRefKPT];
#pragma unroll
  for (int j = 0; j < kRefKPT; ++j) lk[j] = tid + (int64_t)kRefThreads * j < nb ? lk_raw[j] : 0ull;
  auto visit_low = [&](auto f) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kRefKPT; ++j)
      if (lk[j] != 0) f(lk[j]);
  };
  const uint64_t G = block_bound<kRefWaves>(visit_low, (uint32_t)k_eff, (uint32_t)k_eff + 32u, sh.bs);

  // 2. full tiles (next key >= G) in tile order: one pass of 512 tiles at a
  // time, each wave's tiles placed after the earlier waves'
  for (int64_t t0 = 0; t0 < nt; t0 += kRefThreads) {
    const int64_t t = t0 + tid;
    const uint64_t nx = t >= nt ? 0ull : (t0 == 0 ? nx_first : hnext[t]);
    const bool full = nx != 0 && nx >= G;
    const uint64_t m = __ballot(full);
    if (lane == 0) sh.wcnt[wave] = (uint32_t)__popcll(m);
    lds_sync();
    uint32_t before = sh.nfull, tot = 0;
#pragma unroll
    for (int w = 0; w < kRefWaves; ++w) {
      before += w < wave ? sh.wcnt[w] : 0u;
      tot += sh.wcnt[w];
    }
    const uint32_t pos = before + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (full && pos < kRefMaxFull) sh.full_tile[pos] = (uint32_t)t;
    lds_sync();
    if (tid == 0) sh.nfull += tot;
    lds_sync();
  }
  const uint32_t nfull_all = sh.nfull;
  const bool all_rows = nfull_all > kRefMaxFull;  // uniform: then every row is an item
  const int nfull = (int)(all_rows ? 0 : nfull_all);
  // rows of the full tiles (the last tile of the session may be partial and,
  // listed in tile order, is then the last one)
  int64_t full_rows = 0;
  if (nfull > 0) {
    const int64_t tl = sh.full_tile[nfull - 1];
    full_rows = (int64_t)(nfull - 1) * T + ((tl + 1) * T <= n ? T : n - tl * T);
  }
  const int64_t head_items = all_rows ? 0 : nh;
  const int64_t n_items = all_rows ? n : head_items + full_rows;
  if (blockIdx.x == 0 && tid == 0) a.count[sess] = (uint32_t)n_items;
  auto is_full = [&](int64_t t) __attribute__((always_inline)) {  // binary search of the sorted list
    int lo = 0, hi = nfull;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)sh.full_tile[mid] < t) lo = mid + 1; else hi = mid;
    }
    return lo < nfull && (int64_t)sh.full_tile[lo] == t;
  };

  // 3. this wave's items, 64 per round (lane u of round r: item gw + nw
  // (64 r + u)): each lane finds its item's row (-1: no key, stored as 0);
  // the wave then scores the candidates two at a time in lane order, the
  // next pair's row bytes loading while the current pair is scored.
  for (int64_t r0 = 0;; r0 += 64) {
    const int64_t i = gw + (int64_t)nw * (r0 + lane);
    const bool live = i < n_items;
    if (__ballot(live) == 0) break;  // uniform
    int64_t row = -1;
    if (live) {
      if (all_rows) {
        row = i;
      } else if (i < head_items) {
        const uint64_t x = r0 == 0 ? xk : hkey[i];  // rank i / nt of tile i % nt
        if (x != 0 && x >= G && !is_full(i % nt)) row = (int64_t)key_row(x);
      } else {
        const int64_t r = i - head_items;
        row = (int64_t)sh.full_tile[r / T] * T + r % T;
      }
    }
    if (live && row < 0) items[i] = 0ull;
    if constexpr (!EXACT) {  // given scores: every candidate lane at once
      if (row >= 0) items[i] = make_key(S.scores[row], (uint32_t)row);
      continue;
    }
    uint64_t m = __ballot(row >= 0);
    // the rows' bytes: the prefetched ones for lanes 0 and 1 of the first
    // round of head items (their rows are their prefetched keys' rows)
    const bool pre_ok = r0 == 0 && !all_rows;
    // (constant indices into pb: a dynamic index would place it in memory)
    static_assert(kRefPrefetch == 2, "lanes 0 and 1");
    auto bytes_of = [&](int l, int64_t rr) __attribute__((always_inline)) {
      const bool pre = pre_ok && l < kRefPrefetch && gw + (int64_t)nw * l < head_items;
      if (pre) return l == 0 ? pb[0] : pb[1];
      return load_row_bytes(S.idx_rows, rr);
    };
    auto next_pair = [&](int &la, int &lb) __attribute__((always_inline)) {
      la = m ? __builtin_ctzll(m) : -1;
      if (la >= 0) m &= m - 1;
      lb = m ? __builtin_ctzll(m) : -1;
      if (lb >= 0) m &= m - 1;
    };
    int la, lb;
    next_pair(la, lb);
    int64_t ra = la >= 0 ? readlane_i64(row, la) : -1, rb = lb >= 0 ? readlane_i64(row, lb) : -1;
    RowBytes ba = la >= 0 ? bytes_of(la, ra) : RowBytes{}, bb = lb >= 0 ? bytes_of(lb, rb) : RowBytes{};
    while (la >= 0) {  // uniform
      int lc, ld;
      next_pair(lc, ld);
      const int64_t rc = lc >= 0 ? readlane_i64(row, lc) : -1, rd = ld >= 0 ? readlane_i64(row, ld) : -1;
      const RowBytes bc = lc >= 0 ? load_row_bytes(S.idx_rows, rc) : RowBytes{};
      const RowBytes bd = ld >= 0 ? load_row_bytes(S.idx_rows, rd) : RowBytes{};
      if (lb >= 0) {
        const RowBytes rbs[2] = {ba, bb};
        float f[2];
        exact_scores<2>(rbs, H, sh, f);
        if (lane == la) items[i] = make_key(f[0], (uint32_t)ra);
        if (lane == lb) items[i] = make_key(f[1], (uint32_t)rb);
      } else {
        const float f = exact_score(ba, H, sh);
        if (lane == la) items[i] = make_key(f, (uint32_t)ra);
      }
      la = lc; lb = ld; ra = rc; rb = rd; ba = bc; bb = bd;
    }
  }
  if (a.attn_q) {  // the attention query split share
    uint4 *dst = a.attn_q + (size_t)sess * kAttnQVecs;
    if (qt0 + tid < qt1) attn_q_store(qx, a.n_attn_heads, dst, qt0 + tid);
    for (int t = qt0 + tid + kRefThreads; t < qt1; t += kRefThreads) attn_q_split_task(S.q_attn, a.n_attn_heads, dst, t);
  }
}

hipError_t launch_refine(const RefineJob &job, hipStream_t st) {
  RefineArgs a;
  int64_t max_rows = 0;
  for (int i = 0; i < job.n_sessions; ++i) {
    a.s[i] = RefineSession{job.idx_rows[i], job.q[i], job.w[i], job.scores[i], job.q_attn[i], job.n_rows[i], job.hd[i]};
    max_rows = job.n_rows[i] > max_rows ? job.n_rows[i] : max_rows;
  }
  a.hkey = job.hkey;
  a.hlow = job.hlow;
  a.hnext = job.hnext;
  a.items = job.items;
  a.count = job.count;
  a.attn_q = job.attn_q;
  a.n_attn_heads = job.n_attn_heads;
  a.heads_stride = job.heads_stride;
  a.tiles_stride = job.tiles_stride;
  a.items_stride = job.items_stride;
  a.tile_rows = job.tile_rows;
  a.n_idx_heads = job.n_idx_heads;
  a.k = job.k;
  a.mode = (int)job.mode;
  if (max_rows == 0 && (job.mode == RefineJob::kAll || job.mode == RefineJob::kKeysAll)) return hipSuccess;
  const dim3 grid((unsigned)job.blocks, (unsigned)job.n_sessions);
  if (job.mode == RefineJob::kArray)
    refine_kernel<false><<<grid, kRefThreads, 0, st>>>(a);
  else
    refine_kernel<true><<<grid, kRefThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa
