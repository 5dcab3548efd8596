// csa_merge.hip -- the global exact top-k of a session (DS4X page, "CSA
// score/top-512 fusion": the model's exact top-512 with the same float score
// order and lower-index tie break as a separate top-k pass), and optionally
// the attention of the selected rows.
//
// Input: the session's items (csa_refine.hip): exact keys of every row that
// can reach the top-k (plus 0 = "no key" slots), count[session] of them.
// Every workgroup of a session (grid.x = slices) runs the same selection:
//   1. G: a lower bound on the k_eff-th largest key, found with histogram
//      passes (block_bound): at least k_eff keys are >= G, and at most
//      kSelTarget are (or exactly k_eff); the top-k lies among the keys >= G.
//      With at most kSelRankAll keys G admits them all (ranking that many
//      costs less than the passes).
//   2. Candidates = keys >= G.  If they overflow the LDS buffer (many ties,
//      crowded winners), the exact k_eff-th key among them replaces G.
//   3. The candidates are ranked exactly (rank = number of larger
//      candidates).  Workgroup b ranks the candidates whose row hashes to
//      slice b and writes sel_idx[rank] / sel_score[rank] for ranks < k_eff.
//      With attention, the slices are the kAttnGroups row groups and four
//      workgroups (one per 16-head group) share each: all four rank the
//      row group's candidates, the first writes the selection, and each runs
//      the attention of those rows in rank order for its heads and writes
//      their partial (csa_attn.hpp; the same partials as csa_sparse_attn's).
//      A selected candidate's place in that order is the number of the row
//      group's candidates with a larger key (each of them is selected too),
//      found while ranking, so no sort follows.
// Selection keys are (ord32(score) << 32) | (2^32 - 1 - row): distinct,
// larger = better; 0 means "no key".
#include "csa_attn.hpp"
#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "csa_select.hpp"

namespace csa {

constexpr int kSelThreads = kAttnThreads;  // 512
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelKPT = 8;                            // keys per thread in registers
constexpr int kSelRegKeys = kSelThreads * kSelKPT;   // 4096
constexpr int kSelCap = 4096;                         // candidates held in LDS
constexpr int kSelTarget = 1024;                      // candidates at which G is good enough
constexpr int kSelRankAll = 1024;  // at most this many keys: all are ranked (no bound passes)
static_assert(kSelRankAll <= kSelCap, "the candidates fit the LDS buffer");

struct SelSessionArgs {
  const float *scores;  // csa_topk: the given scores (sel_score returns their values)
  int32_t *sel_idx;
  float *sel_score;
  const uint8_t *kv_rows;
  int64_t n_rows;
};

struct SelArgs {
  SelSessionArgs s[CSA_MAX_SESSIONS];
  const uint64_t *items;  // [session][items_stride]
  const uint32_t *count;  // [session]
  const uint4 *attn_q;
  float *attn_part;
  float *attn_ml;
  int64_t items_stride;
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
      BoundShared<kSelWaves> bs;
      uint16_t mine[kSelCap];
    } s;
    AttnStage st;  // used after the ranks are written
  } u;
  int32_t loc_row[CSA_TOPK], ordered[CSA_TOPK];
  uint32_t ccnt, nmine, nloc;
};
// The early stage's rows are copied in while the group list (mine) is
// still read; its logit tiles are written only after that, and may overlap it.
static_assert(kEarlyStageOff + offsetof(AttnStage, lgp) <= offsetof(SelShared, u.s.mine) - offsetof(SelShared, u),
              "the early stage's rows end before the group list");
static_assert(kEarlyStageOff + sizeof(AttnStage) <= sizeof(SelShared::u), "the early stage fits the union");

// Row of a key -> workgroup of the session that ranks it.
__device__ __forceinline__ uint32_t row_slice(uint32_t row, int slices) {
  return (uint32_t)(((uint64_t)(row * 0x9E3779B1u) * (uint32_t)slices) >> 32);
}

template <bool ATTN>
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

  const uint64_t *items = a.items + (size_t)sess * a.items_stride;
  const int64_t ni = (int64_t)a.count[sess];
  // keys in registers: slot j of thread tid is item tid + 512 j.  The first
  // kSelRegKeys slots of the session's item array are read without waiting
  // for the count (the loads stay inside the array; slots past the count
  // hold stale keys and are masked once it has arrived)
  uint64_t h[kSelKPT];
#pragma unroll
  for (int j = 0; j < kSelKPT; ++j) {
    const int64_t i = tid + (int64_t)kSelThreads * j;
    h[j] = items[i < a.items_stride ? i : a.items_stride - 1];
  }
  const bool reg = ni <= kSelRegKeys;  // uniform
  if (tid == 0) { sh.ccnt = 0; sh.nmine = 0; sh.nloc = 0; }
#pragma unroll
  for (int j = 0; j < kSelKPT; ++j) h[j] = tid + (int64_t)kSelThreads * j < ni ? h[j] : 0ull;
  // the candidates >= lb, in batches of 8 slots per thread: fb(ok[8], x[8])
  // in control flow uniform over the wave
  auto scan = [&](uint64_t lb, auto fb) __attribute__((always_inline)) {
    if (reg) {
      bool ok[8];
      uint64_t x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        x[u] = h[u];
        ok[u] = x[u] != 0 && x[u] >= lb;
      }
      fb(ok, x);
    } else {
      for (int64_t i0 = 0; i0 < ni; i0 += (int64_t)kSelThreads * 8) {
        bool ok[8];
        uint64_t x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t i = i0 + tid + (int64_t)kSelThreads * u;
          const uint64_t z = items[i < ni ? i : ni - 1];
          x[u] = i < ni ? z : 0ull;
          ok[u] = x[u] != 0 && x[u] >= lb;
        }
        fb(ok, x);
      }
    }
  };
  auto visit_all = [&](auto f) __attribute__((always_inline)) {
    scan(1ull, [&](const bool (&ok)[8], const uint64_t (&x)[8]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (ok[u]) f(x[u]);
    });
  };

  // 1. the bound G
  const uint64_t G =
      block_bound<kSelWaves>(visit_all, (uint32_t)k_eff, (uint32_t)kSelTarget, sh.u.s.bs, (uint32_t)kSelRankAll);

  // 2. candidates: one LDS atomic per wave and batch, the wave's selected
  // slots taking consecutive positions
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
  scan(G, append);
  __syncthreads();
  int C = (int)sh.ccnt;
  if (C > kSelCap) {
    // too many candidates: the exact k_eff-th key among them
    auto visit_cand = [&](auto f) __attribute__((always_inline)) {
      scan(G, [&](const bool (&ok)[8], const uint64_t (&x)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (ok[u]) f(x[u]);
      });
    };
    const uint64_t thr = block_bound<kSelWaves>(visit_cand, (uint32_t)k_eff, (uint32_t)k_eff, sh.u.s.bs);
    if (tid == 0) sh.ccnt = 0;
    __syncthreads();
    scan(thr, append);
    __syncthreads();
    C = (int)sh.ccnt;
  }

  // 3. rank this workgroup's candidates
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
  // wave w ranks group entries w, w + 8, w + 16, ... up to four per pass
  // over the candidates (the entries of one pass are uniform over the
  // wave).  With attention, a selected entry's position in the group's key
  // order is the number of group entries with a larger key (every such
  // entry has a smaller rank, so it is selected too): the selected rows land
  // in ordered[0..nl) in rank order directly.
  constexpr int kRankPer = 4;
  for (int m0 = wave; m0 < nm; m0 += kRankPer * kSelWaves) {
    uint64_t x[kRankPer];
    bool has[kRankPer];
#pragma unroll
    for (int t = 0; t < kRankPer; ++t) {
      const int m = m0 + kSelWaves * t;
      has[t] = m < nm;  // uniform
      x[t] = has[t] ? sh.u.s.cand[sh.u.s.mine[m]] : ~0ull;  // (all ones: no candidate is larger)
    }
    uint32_t r[kRankPer] = {}, pos[kRankPer] = {};
    for (int j0 = 0; j0 < C; j0 += 4 * 64) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + 64 * u + lane;
        const uint64_t y = sh.u.s.cand[j];
#pragma unroll
        for (int t = 0; t < kRankPer; ++t) r[t] += (uint32_t)__popcll(__ballot(j < C && y > x[t]));
      }
    }
    if constexpr (ATTN) {  // positions in the group's key order
      for (int j0 = 0; j0 < nm; j0 += 64) {
        const int j = j0 + lane;
        const uint64_t y = j < nm ? sh.u.s.cand[sh.u.s.mine[j]] : 0ull;
#pragma unroll
        for (int t = 0; t < kRankPer; ++t) pos[t] += (uint32_t)__popcll(__ballot(y > x[t]));
      }
    }
#pragma unroll
    for (int t = 0; t < kRankPer; ++t) {
      if (lane == 0 && has[t] && r[t] < (uint32_t)k_eff) {
        const uint32_t row = key_row(x[t]);
        if (writer) {
          sel_idx[r[t]] = (int32_t)row;
          if (sel_score) {
            if constexpr (ATTN)  // the fused path: the key holds the score
              sel_score[r[t]] = key_score(x[t]);
            else
              sel_score[r[t]] = a.array_scores ? scores[row] : key_score(x[t]);
          }
        }
        if constexpr (ATTN) {
          sh.ordered[pos[t]] = (int32_t)row;
          atomicAdd(&sh.nloc, 1u);
        }
      }
    }
  }
  if constexpr (!ATTN) return;

  // 4. attention over this workgroup's selected rows, in rank order
  __syncthreads();
  const int nl = (int)sh.nloc;
  attn_group_rows(a.attn_q + (size_t)sess * kAttnQVecs, sh.u.st, sh.ordered, nl, a.s[sess].kv_rows, a.softmax_scale, a.n_heads,
                  hgroup, a.attn_part + (size_t)sess * kAttnPartFloats + (size_t)myslice * CSA_MAX_HEADS * kKvDim,
                  a.attn_ml + (size_t)sess * kAttnMlFloats + (size_t)myslice * CSA_MAX_HEADS * 2);
}

hipError_t launch_select(const SelectJob &job, hipStream_t st) {
  SelArgs a;
  for (int i = 0; i < job.n_sessions; ++i)
    a.s[i] = SelSessionArgs{job.scores[i], job.sel_idx[i], job.sel_score[i],
                            job.attn_part ? job.kv_rows[i] : nullptr, job.n_rows[i]};
  a.items = job.items;
  a.count = job.count;
  a.items_stride = job.items_stride;
  a.attn_q = job.attn_q;
  a.attn_part = job.attn_part;
  a.attn_ml = job.attn_ml;
  a.k = job.k;
  a.n_heads = job.n_heads;
  a.softmax_scale = job.softmax_scale;
  a.array_scores = job.array_scores ? 1 : 0;
  const dim3 grid((unsigned)job.slices, (unsigned)job.n_sessions);
  if (job.attn_part)
    select_kernel<true><<<grid, kSelThreads, 0, st>>>(a);
  else
    select_kernel<false><<<grid, kSelThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa
