// csa_merge.hip -- the global exact top-k of a session from its tiles' heads
// (DS4X page, "CSA score/top-512 fusion": merge the per-tile selections into
// the model's exact top-512 with the same float order and lower-index tie
// break as a separate top-k pass), and optionally the attention of
// the selected rows.
//
// Every workgroup of a session (grid.x = slices) runs the same selection:
//   1. G: a lower bound on the 512th-largest head, found with one or two
//      histogram passes over the heads: at least 512 heads are >= G, and at
//      most kSelTarget are (or exactly 512).  Since every head is a key, at
//      least 512 keys are >= G, so G also bounds the global 512th key, and
//      the top-k (k <= 512) lies among the keys >= G.
//   2. A tile is "full" when its hd-th (smallest) head is >= G: it may hold
//      keys >= G that are not heads.  Any other tile holds no key >= G beyond
//      its heads.  Candidates = heads >= G of tiles that are not full, plus
//      every key >= G of the full tiles, read from the score array.  (Few
//      heads per tile hold at least hd keys >= G, so at most kSelTarget / hd
//      tiles are full.)
//   3. If the candidates overflow the LDS buffer (many ties, crowded
//      winners), the exact k_eff-th key among them replaces G.
//   4. The candidates are ranked exactly (rank = number of larger
//      candidates).  Workgroup b ranks the candidates whose row hashes to
//      slice b and writes sel_idx[rank] / sel_score[rank] for ranks < k_eff.
//      With attention, the slices are the kAttnGroups row groups and four
//      workgroups (one per 16-head group) share each: all four rank the
//      row group's candidates, the first writes the selection, and each runs
//      the attention of those rows in rank order for its heads and writes
//      their partial (csa_attn.hpp; the same partials as csa_sparse_attn's).
// Selection keys are (ord32(score) << 32) | (2^32 - 1 - row): distinct,
// larger = better; 0 means "no key".
#include "csa_attn.hpp"
#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "csa_select.hpp"

namespace csa {

constexpr int kSelThreads = kAttnThreads;  // 512
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelKPT = 8;                            // heads per thread in registers
constexpr int kSelRegHeads = kSelThreads * kSelKPT;  // 4096
constexpr int kSelBins = 2 * kSelThreads;             // histogram bins per pass
constexpr int kSelCap = 4096;                         // candidates held in LDS
constexpr int kSelTarget = 1024;                      // candidates at which G is good enough
constexpr int kSelMaxFull = kSelTarget / kMinTileHeads;  // full tiles listed (each holds >= hd heads >= G)

struct SelSessionArgs {
  const float *scores;
  int32_t *sel_idx;
  float *sel_score;
  const uint8_t *kv_rows;
  int64_t n_rows;
  int hd;
};

struct SelArgs {
  SelSessionArgs s[CSA_MAX_SESSIONS];
  const uint64_t *heads;
  const uint4 *attn_q;
  float *attn_part;
  float *attn_ml;
  int64_t heads_stride;
  int tile_rows;
  int k;
  int n_heads;
  float softmax_scale;
  int array_scores;
};
static_assert(sizeof(SelArgs) <= 4096, "kernel argument block");

// The early attention stage (at most k_eff <= 512 candidates, read with the
// rank scan's slack) starts this many bytes into the selection union.
constexpr int kEarlyStageOff = 8192;
static_assert((CSA_TOPK + 4 * 64) * 8 <= kEarlyStageOff, "the stage leaves the live candidates alone");

struct SelShared {
  union {
    struct {
      uint64_t cand[kSelCap + 4 * 64];  // + over-read slack of the rank scan
      uint32_t hist[kSelBins];
      uint16_t mine[kSelCap];
    } s;
    AttnStage st;  // used after the ranks are written
  } u;
  uint64_t red_lo[kSelWaves], red_hi[kSelWaves];
  uint32_t red_n[kSelWaves];
  uint32_t full_list[kSelMaxFull];
  int32_t loc_rank[CSA_TOPK + 16], loc_row[CSA_TOPK], ordered[CSA_TOPK];
  uint32_t ccnt, nfull, nmine, nloc;
  uint32_t bin, ca, cb;
};
// The early stage's rows are copied in while the group list (mine) is
// still read; its logit tiles are written only after that, and may overlap it.
static_assert(kEarlyStageOff + offsetof(AttnStage, lgp) <= offsetof(SelShared, u.s.mine) - offsetof(SelShared, u),
              "the early stage's rows end before the group list");
static_assert(kEarlyStageOff + sizeof(AttnStage) <= sizeof(SelShared::u), "the early stage fits the union");

// Lower bound G on the need-th largest of the keys that `visit` enumerates
// (every thread visits its share, calling f(key) for each nonzero key): at
// least need keys are >= G, and at most max(target, need) are, unless the
// finest bin already holds more.  Returns 1 (every key) when there are at
// most need keys.  All threads call it.
template <class Visit>
__device__ __forceinline__ uint64_t sel_bound(Visit visit, uint32_t need, uint32_t target, SelShared &sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  auto umin = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
  auto umax = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  auto uadd = [](uint32_t a, uint32_t b) { return a + b; };
  // range of the score parts (key >> 32), and the count
  uint32_t mn = ~0u, mx = 0;
  uint32_t cnt = 0;
  visit([&](uint64_t x) __attribute__((always_inline)) {
    const uint32_t o = (uint32_t)(x >> 32);
    mn = o < mn ? o : mn;
    mx = o > mx ? o : mx;
    ++cnt;
  });
  mn = wave_reduce_u32(mn, ~0u, umin);
  mx = wave_reduce_u32(mx, 0u, umax);
  cnt = wave_reduce_u32(cnt, 0u, uadd);
  if (lane == 0) { sh.red_lo[wave] = mn; sh.red_hi[wave] = mx; sh.red_n[wave] = cnt; }
  // the first pass's histogram is cleared under the same barrier (visit
  // reads nothing of it); red_n is next written after the pass's atomics
  // and their barrier, which every thread reaches only after reading it here
  for (int i = tid; i < kSelBins; i += kSelThreads) sh.u.s.hist[i] = 0;
  __syncthreads();
  uint32_t omin = ~0u, omax = 0;
  uint32_t total = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    omin = (uint32_t)sh.red_lo[w] < omin ? (uint32_t)sh.red_lo[w] : omin;
    omax = (uint32_t)sh.red_hi[w] > omax ? (uint32_t)sh.red_hi[w] : omax;
    total += sh.red_n[w];
  }
  uint64_t lo = (uint64_t)omin << 32, hi = ((uint64_t)omax << 32) | 0xFFFFFFFFull;
  if (total <= need) return 1ull;
  // (even with few keys, G = the smallest would make every tile "full")
  uint32_t above = 0;  // keys above the current range [lo, hi]
  for (bool first = true;; first = false) {
    const uint64_t span = hi - lo;
    const int hb = span ? 63 - __clzll((long long)span) : 0;
    const int shift = hb > 9 ? hb - 9 : 0;  // span >> shift < kSelBins (1024)
    if (!first) {
      for (int i = tid; i < kSelBins; i += kSelThreads) sh.u.s.hist[i] = 0;
      __syncthreads();
    }
    visit([&](uint64_t x) __attribute__((always_inline)) {
      if (x >= lo && x <= hi) atomicAdd(&sh.u.s.hist[(uint32_t)((x - lo) >> shift)], 1u);
    });
    __syncthreads();
    const uint32_t need_here = need - above;
    // thread t owns the upper bin kSelBins-1-2t and the lower bin
    // kSelBins-2-2t, so "bins above" is a prefix over threads
    const uint32_t bu = kSelBins - 1 - 2 * tid;
    const uint32_t h1 = sh.u.s.hist[bu], h0 = sh.u.s.hist[bu - 1];
    const uint32_t s = h0 + h1;
    const uint32_t incl = wave_scan_u32(s, 0u, uadd);
    if (lane == 63) sh.red_n[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += sh.red_n[w];
    const uint32_t X = incl - s + before;  // keys in bins above bu
    if (X < need_here && need_here <= X + h1) {
      sh.bin = bu; sh.ca = X; sh.cb = h1;
    } else if (X + h1 < need_here && need_here <= X + s) {
      sh.bin = bu - 1; sh.ca = X + h1; sh.cb = h0;
    }
    __syncthreads();
    const uint32_t b = sh.bin, ca = sh.ca, cb = sh.cb;
    const uint64_t gb = lo + ((uint64_t)b << shift);
    // (uniform; after the return nothing writes bin, ca, cb or the
    // histogram before another barrier)
    if (above + ca + cb <= target || shift == 0) return gb;
    __syncthreads();  // every thread has read bin, ca, cb
    above += ca;
    const uint64_t top = gb + ((1ull << shift) - 1);
    lo = gb;
    hi = top < hi ? top : hi;
  }
}

// Row of a key -> workgroup of the session that ranks it.
__device__ __forceinline__ uint32_t row_slice(uint32_t row, int slices) {
  return (uint32_t)(((uint64_t)(row * 0x9E3779B1u) * (uint32_t)slices) >> 32);
}

// REG: every session's heads fit in registers (at most kSelRegHeads), chosen
// on the host for the whole launch; otherwise they are re-read per pass.
template <bool ATTN, bool REG>
__global__ void __launch_bounds__(kSelThreads) select_kernel(const SelArgs a) {
  const int sess = blockIdx.y;
  // fields used inside lambdas are copied first: a lambda taking the address
  // of the kernel argument block would force a private copy of it
  const float *const scores = a.s[sess].scores;
  int32_t *const sel_idx = a.s[sess].sel_idx;
  float *const sel_score = a.s[sess].sel_score;
  const int64_t n = a.s[sess].n_rows;
  const int k = a.k;
  const int k_eff = (int)(n < k ? n : k);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __shared__ SelShared sh;

  if (blockIdx.x == 0)
    for (int r = k_eff + tid; r < k; r += kSelThreads) {
      sel_idx[r] = -1;
      if (sel_score) sel_score[r] = -__builtin_inff();
    }
  // ATTN: workgroup b ranks (and attends over) the rows of row group
  // b % kAttnGroups, for head group b / kAttnGroups; the head-group-0
  // workgroups write the selection
  const int nslice = ATTN ? kAttnGroups : (int)gridDim.x;
  const uint32_t myslice = ATTN ? blockIdx.x % kAttnGroups : blockIdx.x;
  const int hgroup = ATTN ? (int)(blockIdx.x / kAttnGroups) : 0;
  const bool writer = hgroup == 0;
  // the attention query terms of this workgroup's head group, loaded now so
  // they arrive during the selection
  AttnQuery aq;
  if constexpr (ATTN) load_attn_query(aq, a.attn_q + (size_t)sess * kAttnQVecs, hgroup);
  if (k_eff == 0) {
    if constexpr (ATTN) {  // an empty group partial: m = -inf, l = 0
      float *ml = a.attn_ml + (size_t)sess * kAttnMlFloats + (size_t)myslice * CSA_MAX_HEADS * 2;
      const int h = 16 * hgroup + tid;
      if (tid < 16 && h < a.n_heads) {
        ml[2 * h] = -__builtin_inff();
        ml[2 * h + 1] = 0.0f;
      }
    }
    return;
  }

  const int T = a.tile_rows;
  const int hd = a.s[sess].hd;
  const int lT = __builtin_ctz((unsigned)T), lhd = __builtin_ctz((unsigned)hd);  // both powers of two
  const int64_t nt = (n + T - 1) >> lT;
  const int64_t nh = nt * hd;
  const uint64_t *heads = a.heads + (size_t)sess * a.heads_stride;
  constexpr bool reg = REG;
  if (tid == 0) { sh.ccnt = 0; sh.nfull = 0; sh.nmine = 0; sh.nloc = 0; }

  // heads in registers: slot j of thread tid is head tid + 1024 j
  uint64_t h[kSelKPT];
  if constexpr (reg) {
#pragma unroll
    for (int j = 0; j < kSelKPT; ++j) {
      const int64_t i = tid + (int64_t)kSelThreads * j;
      const uint64_t y = heads[i < nh ? i : nh - 1];  // clamped: no branch around the load
      h[j] = i < nh ? y : 0ull;
    }
  }
  // every head slot of this thread, in control flow uniform over the wave:
  // f(ok, x), ok = "x is a head"
  auto scan_heads = [&](auto f) __attribute__((always_inline)) {
    if constexpr (reg) {
#pragma unroll
      for (int j = 0; j < kSelKPT; ++j) f(h[j] != 0, h[j]);
    } else {
      for (int64_t i0 = 0; i0 < nh; i0 += (int64_t)kSelThreads * 8) {
        uint64_t y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t i = i0 + tid + (int64_t)kSelThreads * u;
          const uint64_t z = heads[i < nh ? i : nh - 1];
          y[u] = i < nh ? z : 0ull;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) f(y[u] != 0, y[u]);
      }
    }
  };
  auto visit_heads = [&](auto f) __attribute__((always_inline)) {
    scan_heads([&](bool ok, uint64_t x) __attribute__((always_inline)) {
      if (ok) f(x);
    });
  };

  // 1. the bound G
  const uint64_t G = sel_bound(visit_heads, (uint32_t)kTopK, (uint32_t)kSelTarget, sh);

  // 2. full tiles (hd-th head >= G) and the candidates
  auto tile_is_full = [&](int64_t t) __attribute__((always_inline)) {
    const uint64_t last = heads[t * hd + hd - 1];
    return last != 0 && last >= G;
  };
  // REG: a tile's hd heads sit in hd consecutive lanes of one slot (hd
  // divides 64), so the lane of its last head decides "full" for all of
  // them with one ballot, and lists the tile
  bool fullbit[kSelKPT];
  if constexpr (reg) {
    bool lists[kSelKPT];
    uint64_t lm[kSelKPT];
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < kSelKPT; ++j) {
      const int i = tid + kSelThreads * j;  // < kSelRegHeads
      lists[j] = i < nh && (i & (hd - 1)) == hd - 1 && h[j] != 0 && h[j] >= G;
      lm[j] = __ballot(lists[j]);
      fullbit[j] = ((lm[j] >> (lane | (hd - 1))) & 1ull) != 0;
      tot += (uint32_t)__popcll(lm[j]);
    }
    if (tot != 0) {  // one LDS atomic per wave
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&sh.nfull, tot);
      base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
#pragma unroll
      for (int j = 0; j < kSelKPT; ++j) {
        const uint32_t p = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(lm[j] >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)lm[j], 0u));
        if (lists[j] && p < kSelMaxFull) sh.full_list[p] = (uint32_t)((tid + kSelThreads * j) >> lhd);
        base += (uint32_t)__popcll(lm[j]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSelKPT; ++j) fullbit[j] = false;
    for (int64_t t = tid; t < nt; t += kSelThreads)
      if (tile_is_full(t)) {
        const uint32_t p = atomicAdd(&sh.nfull, 1u);
        if (p < kSelMaxFull) sh.full_list[p] = (uint32_t)t;
      }
  }

  // candidates >= lb, in batches of 8 slots per thread: fb(ok[8], x[8]) in
  // control flow uniform over the wave.  Heads of tiles that are not full:
  auto scan_head_cand = [&](uint64_t lb, auto fb) __attribute__((always_inline)) {
    if constexpr (reg) {
#pragma unroll
      for (int j0 = 0; j0 < kSelKPT; j0 += 8) {
        bool ok[8];
        uint64_t x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          x[u] = h[j0 + u];
          ok[u] = x[u] != 0 && x[u] >= lb && !fullbit[j0 + u];
        }
        fb(ok, x);
      }
    } else {
      for (int64_t i0 = 0; i0 < nh; i0 += (int64_t)kSelThreads * 8) {
        bool ok[8];
        uint64_t x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t i = i0 + tid + (int64_t)kSelThreads * u;
          const uint64_t z = heads[i < nh ? i : nh - 1];
          x[u] = i < nh ? z : 0ull;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          // the tile of a head: keys carry the row, tiles are T rows
          const int64_t t = x[u] != 0 ? (int64_t)(key_row(x[u]) >> lT) : 0;
          ok[u] = x[u] != 0 && x[u] >= lb && !tile_is_full(t);
        }
        fb(ok, x);
      }
    }
  };
  // ... and every key of the full tiles (sh.full_list[0..nfull) complete)
  auto scan_full_rows = [&](int nfull, uint64_t lb, auto fb) __attribute__((always_inline)) {
    const int nfr = nfull << lT;  // at most kSelMaxFull * 4096
    for (int i0 = 0; i0 < nfr; i0 += kSelThreads * 8) {
      float v[8];
      int64_t row[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + tid + kSelThreads * u;
        row[u] = i < nfr ? ((int64_t)sh.full_list[i >> lT] << lT) + (i & (T - 1)) : n;
        v[u] = scores[row[u] < n ? row[u] : n - 1];
      }
      bool ok[8];
      uint64_t x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        x[u] = ((uint64_t)score_ord(v[u]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)row[u]);
        ok[u] = row[u] < n && x[u] >= lb;
      }
      fb(ok, x);
    }
  };
  // one LDS atomic per wave and batch: the wave's selected slots take
  // consecutive positions
  auto append = [&](const bool (&ok)[8], const uint64_t (&x)[8]) __attribute__((always_inline)) {
    uint64_t m[8];
    uint32_t tot = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      m[u] = __ballot(ok[u]);
      tot += (uint32_t)__popcll(m[u]);
    }
    if (tot == 0) return;
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&sh.ccnt, tot);
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t p =
          base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m[u] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[u], 0u));
      if (ok[u] && p < (uint32_t)kSelCap) sh.u.s.cand[p] = x[u];
      base += (uint32_t)__popcll(m[u]);
    }
  };
  scan_head_cand(G, append);
  __syncthreads();  // full tiles listed, head candidates appended
  const int nfull = (int)(sh.nfull < kSelMaxFull ? sh.nfull : kSelMaxFull);
  if (nfull > 0) {  // uniform
    scan_full_rows(nfull, G, append);
    __syncthreads();
  }
  int C = (int)sh.ccnt;
  if (C > kSelCap) {
    // 3. too many candidates: the exact k_eff-th key among them
    auto visit_cand = [&](auto f) __attribute__((always_inline)) {
      auto each = [&](const bool (&ok)[8], const uint64_t (&x)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (ok[u]) f(x[u]);
      };
      scan_head_cand(G, each);
      scan_full_rows(nfull, G, each);
    };
    const uint64_t thr = sel_bound(visit_cand, (uint32_t)k_eff, (uint32_t)k_eff, sh);
    if (tid == 0) sh.ccnt = 0;
    __syncthreads();
    scan_head_cand(thr, append);
    scan_full_rows(nfull, thr, append);
    __syncthreads();
    C = (int)sh.ccnt;
  }

  // 4. rank this workgroup's candidates
  for (int i0 = 0; i0 < C; i0 += kSelThreads) {
    const int i = i0 + tid;
    if (i < C && row_slice(key_row(sh.u.s.cand[i]), nslice) == myslice) sh.u.s.mine[atomicAdd(&sh.nmine, 1u)] = (uint16_t)i;
  }
  __syncthreads();
  const int nm = (int)sh.nmine;
  if constexpr (ATTN) {
    if (C <= k_eff && nm <= kRawRows) {  // uniform
      // C >= k_eff always (G bounds the k_eff-th key), so here every
      // candidate is selected: the row group attends over its candidates in
      // key order (= rank order).  Their rows are staged while that order
      // and the global ranks are formed; the stage sits in the union past
      // the live candidates and before the group list.
      AttnStage &est = *reinterpret_cast<AttnStage *>(reinterpret_cast<char *>(&sh.u) + kEarlyStageOff);
      if (tid < nm) sh.loc_row[tid] = (int32_t)key_row(sh.u.s.cand[sh.u.s.mine[tid]]);
      __syncthreads();
      attn_stage_dma_issue(a.s[sess].kv_rows, sh.loc_row, nm, est.raw);
      if (wave == 0) {  // slot i (candidate mine[i]) -> its position in the group's key order
        const uint64_t x = lane < nm ? sh.u.s.cand[sh.u.s.mine[lane]] : 0ull;
        const uint32_t xlo = (uint32_t)x, xhi = (uint32_t)(x >> 32);
        int pos = 0;
        for (int j = 0; j < nm; ++j) {
          const uint64_t y = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)xhi, j) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane((int)xlo, j);
          pos += y > x ? 1 : 0;
        }
        if (lane < nm) sh.ordered[pos] = lane;
      }
      // the global ranks: the row group's four workgroups split its
      // candidates by row index (each workgroup lists and numbers its
      // candidates in its own order), waves taking list entries in turn
      for (int i = wave; i < nm; i += kSelWaves) {
        const uint64_t x = sh.u.s.cand[sh.u.s.mine[i]];
        if ((int)(key_row(x) % kAttnHeadGroups) != hgroup) continue;  // uniform over the wave
        uint32_t r = 0;
        for (int j0 = 0; j0 < C; j0 += 4 * 64) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int j = j0 + 64 * u + lane;
            const uint64_t y = sh.u.s.cand[j];
            r += (uint32_t)__popcll(__ballot(j < C && y > x));
          }
        }
        if (lane == 0) {
          sel_idx[r] = (int32_t)key_row(x);
          if (sel_score) sel_score[r] = key_score(x);
        }
      }
      wait_vmcnt<0>();  // this wave's row copies have landed
      __syncthreads();
      attn_stage_dma_finish(a.s[sess].kv_rows, sh.loc_row, nm, est.raw);
      __syncthreads();
      attn_staged_rows(aq, est, sh.ordered, nm, a.softmax_scale, a.n_heads, hgroup,
                       a.attn_part + (size_t)sess * kAttnPartFloats + (size_t)myslice * CSA_MAX_HEADS * kKvDim,
                       a.attn_ml + (size_t)sess * kAttnMlFloats + (size_t)myslice * CSA_MAX_HEADS * 2);
      return;
    }
  }
  // warm the L2 with the KV rows of this workgroup's candidates (a superset
  // of the rows it will attend over) while the ranks are computed
  uint32_t warm = 0;
  if constexpr (ATTN) {
    const uint8_t *kv = a.s[sess].kv_rows;
    for (int t = tid; t < nm * 6; t += kSelThreads) {
      const uint32_t row = key_row(sh.u.s.cand[sh.u.s.mine[t / 6]]);
      const int off = 128 * (t % 6) < kKvRowBytes - 1 ? 128 * (t % 6) : kKvRowBytes - 1;
      warm ^= kv[(size_t)row * kKvRowBytes + off];
    }
  }
  for (int m = wave; m < nm; m += kSelWaves) {
    const uint64_t x = sh.u.s.cand[sh.u.s.mine[m]];
    uint32_t r = 0;
    for (int j0 = 0; j0 < C; j0 += 4 * 64) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + 64 * u + lane;
        const uint64_t y = sh.u.s.cand[j];
        r += (uint32_t)__popcll(__ballot(j < C && y > x));
      }
    }
    if (lane == 0 && r < (uint32_t)k_eff) {
      const uint32_t row = key_row(x);
      if (writer) {
        sel_idx[r] = (int32_t)row;
        if (sel_score) {
          if constexpr (ATTN)  // the fused path: the key holds the score
            sel_score[r] = key_score(x);
          else
            sel_score[r] = a.array_scores ? scores[row] : key_score(x);
        }
      }
      const uint32_t p = atomicAdd(&sh.nloc, 1u);
      sh.loc_rank[p] = (int32_t)r;
      sh.loc_row[p] = (int32_t)row;
    }
  }
  if constexpr (!ATTN) return;
  if (warm == 0x5A5A5A5Au && a.k < 0) sel_idx[0] = 0;  // never true (k >= 1): keeps the warming loads

  // 5. attention over this workgroup's selected rows, in rank order
  __syncthreads();
  const int nl = (int)sh.nloc;
  attn_order(sh.loc_rank, sh.loc_row, nl, sh.ordered);
  attn_group_rows(a.attn_q + (size_t)sess * kAttnQVecs, sh.u.st, sh.ordered, nl, a.s[sess].kv_rows, a.softmax_scale, a.n_heads,
                  hgroup, a.attn_part + (size_t)sess * kAttnPartFloats + (size_t)myslice * CSA_MAX_HEADS * kKvDim,
                  a.attn_ml + (size_t)sess * kAttnMlFloats + (size_t)myslice * CSA_MAX_HEADS * 2);
}

hipError_t launch_select(const SelectJob &job, hipStream_t st) {
  SelArgs a;
  for (int i = 0; i < job.n_sessions; ++i)
    a.s[i] = SelSessionArgs{job.scores[i], job.sel_idx[i], job.sel_score[i],
                            job.attn_part ? job.kv_rows[i] : nullptr, job.n_rows[i], job.hd[i]};
  a.heads = job.heads;
  a.attn_q = job.attn_q;
  a.attn_part = job.attn_part;
  a.attn_ml = job.attn_ml;
  a.heads_stride = job.heads_stride;
  a.tile_rows = job.tile_rows;
  a.k = job.k;
  a.n_heads = job.n_heads;
  a.softmax_scale = job.softmax_scale;
  a.array_scores = job.array_scores ? 1 : 0;
  const dim3 grid((unsigned)job.slices, (unsigned)job.n_sessions);
  bool reg = true;
  for (int i = 0; i < job.n_sessions; ++i)
    reg = reg && ((job.n_rows[i] + job.tile_rows - 1) / job.tile_rows) * job.hd[i] <= kSelRegHeads;
  if (job.attn_part) {
    if (reg) select_kernel<true, true><<<grid, kSelThreads, 0, st>>>(a);
    else select_kernel<true, false><<<grid, kSelThreads, 0, st>>>(a);
  } else {
    if (reg) select_kernel<false, true><<<grid, kSelThreads, 0, st>>>(a);
    else select_kernel<false, false><<<grid, kSelThreads, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace csa
