// csa_select.hpp -- workgroup-level exact selection on 64-bit keys.
//
// Keys are (ord(score) << 32) | (2^32 - 1 - row): distinct, larger = better
// (larger score, then lower row index), and every real key is >= 2^31, so 0
// means "no key".  block_kth_largest() is an MSB-first radix select that
// starts at the highest bit in which the candidate keys differ, uses 8-bit
// digits with one LDS histogram per wave, and stops as soon as the keys
// sharing the current prefix are exactly the ones still needed.  The
// helpers communicate through LDS only (lds_sync): global loads a caller
// has in flight stay in flight across their barriers.
#pragma once

#include "csa_device.hpp"

namespace csa {

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, 64);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Cross-lane steps on the DPP network (GFX9 row_shr:n = 0x110 + n,
// row_bcast:15 = 0x142 into rows 1 and 3, row_bcast:31 = 0x143 into rows 2
// and 3).  Lanes without a source keep `ident`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t ident, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive scan of v over the lanes of the wave in lane order with an
// associative op whose identity is ident (lane 63 ends with the total).
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v, uint32_t ident, Op op) {
  v = op(v, dpp_u32<0x111, 0xF>(ident, v));
  v = op(v, dpp_u32<0x112, 0xF>(ident, v));
  v = op(v, dpp_u32<0x114, 0xF>(ident, v));
  v = op(v, dpp_u32<0x118, 0xF>(ident, v));
  v = op(v, dpp_u32<0x142, 0xA>(ident, v));
  v = op(v, dpp_u32<0x143, 0xC>(ident, v));
  return v;
}

template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, uint32_t ident, Op op) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_u32(v, ident, op), 63);
}

template <int NW>  // waves per workgroup
struct SelScratch {
  uint32_t hist[NW][256];
  uint64_t wmax[NW], wmin[NW];
  uint32_t wcnt[NW];
  uint64_t r_max, r_min;
  uint32_t r_cnt;
  int digit;
  uint32_t above, bin;
};

// Wave 0 only: digit d with sum(h[d+1..]) < need <= sum(h[d..]); returns d,
// writes the count above it.
__device__ __forceinline__ int find_digit_wave(const uint32_t *h, uint32_t need, uint32_t *above) {
  const int lane = threadIdx.x & 63;
  const uint32_t c0 = h[4 * lane], c1 = h[4 * lane + 1], c2 = h[4 * lane + 2], c3 = h[4 * lane + 3];
  const uint32_t mine = c0 + c1 + c2 + c3;
  uint32_t suf = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = (uint32_t)__shfl_down((int)suf, off, 64);
    if (lane + off < 64) suf += v;
  }
  const uint32_t after = suf - mine;
  int digit = -1;
  uint32_t ab = 0;
  if (after < need && need <= suf) {
    uint32_t acc = after;
    if (acc + c3 >= need) {
      digit = 4 * lane + 3; ab = acc;
    } else {
      acc += c3;
      if (acc + c2 >= need) {
        digit = 4 * lane + 2; ab = acc;
      } else {
        acc += c2;
        if (acc + c1 >= need) { digit = 4 * lane + 1; ab = acc; }
        else { acc += c1; digit = 4 * lane; ab = acc; }
      }
    }
  }
  const unsigned long long ball = __ballot(digit >= 0);
  const int src = ball ? (int)__ffsll((long long)ball) - 1 : 0;
  *above = (uint32_t)__shfl((int)ab, src, 64);
  return __shfl(digit, src, 64);
}

// Threshold of the k largest keys among {key(i) : i < count, key(i) >= lb}:
// returns thr such that exactly min(k, #valid) valid keys are >= thr (thr >=
// lb).  All NW*64 threads of the workgroup must call it; k >= 1.
template <int NW, class KeyFn>
__device__ uint64_t block_kth_largest(KeyFn key, int count, int k, uint64_t lb, SelScratch<NW> &sc) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int NT = NW * 64;
  uint64_t kmax = 0, kmin = ~0ull;
  uint32_t cnt = 0;
  for (int i = tid; i < count; i += NT) {
    const uint64_t x = key(i);
    if (x >= lb) {
      kmax = x > kmax ? x : kmax;
      kmin = x < kmin ? x : kmin;
      ++cnt;
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const uint64_t a = shfl_xor_u64(kmax, m), b = shfl_xor_u64(kmin, m);
    kmax = a > kmax ? a : kmax;
    kmin = b < kmin ? b : kmin;
    cnt += (uint32_t)__shfl_xor((int)cnt, m, 64);
  }
  if (lane == 0) { sc.wmax[wave] = kmax; sc.wmin[wave] = kmin; sc.wcnt[wave] = cnt; }
  lds_sync();
  if (tid == 0) {
    uint64_t M = 0, m = ~0ull;
    uint32_t c = 0;
    for (int w = 0; w < NW; ++w) {
      M = sc.wmax[w] > M ? sc.wmax[w] : M;
      m = sc.wmin[w] < m ? sc.wmin[w] : m;
      c += sc.wcnt[w];
    }
    sc.r_max = M; sc.r_min = m; sc.r_cnt = c;
  }
  lds_sync();
  const uint32_t total = sc.r_cnt;
  const uint64_t gmax = sc.r_max, gmin = sc.r_min;
  lds_sync();
  if (total <= (uint32_t)k) return lb;
  int hi = 63 - __clzll((long long)(gmax ^ gmin));  // keys are distinct: gmax != gmin
  uint64_t prefix = (hi == 63) ? 0ull : (gmax & ~((2ull << hi) - 1));
  uint32_t need = (uint32_t)k;
  for (;;) {
    const int width = hi + 1 < 8 ? hi + 1 : 8;
    const int shift = hi - width + 1;
    const uint64_t pmask = (hi == 63) ? 0ull : ~((2ull << hi) - 1);
    for (int i = tid; i < NW * 256; i += NT) (&sc.hist[0][0])[i] = 0;
    lds_sync();
    for (int i = tid; i < count; i += NT) {
      const uint64_t x = key(i);
      if (x >= lb && (x & pmask) == prefix) atomicAdd(&sc.hist[wave][(uint32_t)(x >> shift) & 255u], 1u);
    }
    lds_sync();
    for (int b = tid; b < 256; b += NT) {
      uint32_t s = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += sc.hist[w][b];
      sc.hist[0][b] = s;
    }
    lds_sync();
    if (wave == 0) {
      uint32_t above;
      const int d = find_digit_wave(sc.hist[0], need, &above);
      if (lane == 0) { sc.digit = d; sc.above = above; sc.bin = sc.hist[0][d]; }
    }
    lds_sync();
    const int d = sc.digit;
    need -= sc.above;
    prefix |= (uint64_t)d << shift;
    const bool done = (sc.bin == need);
    lds_sync();
    if (done) return prefix > lb ? prefix : lb;
    hi = shift - 1;
  }
}

// Same contract as block_kth_largest, for keys held in registers: each
// thread passes KPT slots of which the first nj (the same in every thread)
// are live; 0 or keys below lb are ignored.  Every pass reads registers
// only; LDS holds just the per-wave histograms.
template <int NW, int KPT>
__device__ uint64_t block_kth_largest_reg(const uint64_t (&x)[KPT], int nj, int k, uint64_t lb,
                                          SelScratch<NW> &sc) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int NT = NW * 64;
  uint64_t kmax = 0, kmin = ~0ull;
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool v = j < nj && x[j] >= lb && x[j] != 0;
    kmax = (v && x[j] > kmax) ? x[j] : kmax;
    kmin = (v && x[j] < kmin) ? x[j] : kmin;
    cnt += v ? 1u : 0u;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const uint64_t a = shfl_xor_u64(kmax, m), b = shfl_xor_u64(kmin, m);
    kmax = a > kmax ? a : kmax;
    kmin = b < kmin ? b : kmin;
    cnt += (uint32_t)__shfl_xor((int)cnt, m, 64);
  }
  if (lane == 0) { sc.wmax[wave] = kmax; sc.wmin[wave] = kmin; sc.wcnt[wave] = cnt; }
  lds_sync();
  uint64_t gmax = 0, gmin = ~0ull;
  uint32_t total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    gmax = sc.wmax[w] > gmax ? sc.wmax[w] : gmax;
    gmin = sc.wmin[w] < gmin ? sc.wmin[w] : gmin;
    total += sc.wcnt[w];
  }
  if (total <= (uint32_t)k) {
    lds_sync();
    return lb;
  }
  int hi = 63 - __clzll((long long)(gmax ^ gmin));
  uint64_t prefix = (hi == 63) ? 0ull : (gmax & ~((2ull << hi) - 1));
  uint32_t need = (uint32_t)k;
  for (;;) {
    const int width = hi + 1 < 8 ? hi + 1 : 8;
    const int shift = hi - width + 1;
    const uint64_t pmask = (hi == 63) ? 0ull : ~((2ull << hi) - 1);
    for (int i = tid; i < NW * 256; i += NT) (&sc.hist[0][0])[i] = 0;
    lds_sync();
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (j < nj && x[j] >= lb && x[j] != 0 && (x[j] & pmask) == prefix)
        atomicAdd(&sc.hist[wave][(uint32_t)(x[j] >> shift) & 255u], 1u);
    }
    lds_sync();
    for (int b = tid; b < 256; b += NT) {
      uint32_t s = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += sc.hist[w][b];
      sc.hist[0][b] = s;
    }
    lds_sync();
    if (wave == 0) {
      uint32_t above;
      const int d = find_digit_wave(sc.hist[0], need, &above);
      if (lane == 0) { sc.digit = d; sc.above = above; sc.bin = sc.hist[0][d]; }
    }
    lds_sync();
    const int d = sc.digit;
    need -= sc.above;
    prefix |= (uint64_t)d << shift;
    const bool done = (sc.bin == need);
    lds_sync();
    if (done) return prefix > lb ? prefix : lb;
    hi = shift - 1;
  }
}

// Scratch of block_bound for a workgroup of NW waves.
template <int NW>
struct BoundShared {
  static constexpr int kBins = 2 * NW * 64;  // two histogram bins per thread
  uint32_t hist[kBins];
  uint32_t red_lo[NW], red_hi[NW], red_n[NW];
  uint32_t bin, ca, cb;
};

// Lower bound G on the need-th largest of the keys that `visit` enumerates
// (every thread visits its share, calling f(key) for each nonzero key): at
// least need keys are >= G, and at most max(target, need) are, unless the
// finest bin already holds more.  Returns 1 (every key) when there are at
// most max(need, all_upto) keys (a caller that handles that many keys as
// cheaply as it narrows them skips the passes).  Histogram passes over the
// key range, 2 NW 64 bins each, narrowing to the bin that holds the need-th
// key.  All threads call it.
template <int NW, class Visit>
__device__ __forceinline__ uint64_t block_bound(Visit visit, uint32_t need, uint32_t target, BoundShared<NW> &sh,
                                                uint32_t all_upto = 0) {
  constexpr int NT = NW * 64, kBins = BoundShared<NW>::kBins;
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
  for (int i = tid; i < kBins; i += NT) sh.hist[i] = 0;
  lds_sync();
  uint32_t omin = ~0u, omax = 0;
  uint32_t total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    omin = sh.red_lo[w] < omin ? sh.red_lo[w] : omin;
    omax = sh.red_hi[w] > omax ? sh.red_hi[w] : omax;
    total += sh.red_n[w];
  }
  uint64_t lo = (uint64_t)omin << 32, hi = ((uint64_t)omax << 32) | 0xFFFFFFFFull;
  if (total <= need || total <= all_upto) return 1ull;
  uint32_t above = 0;  // keys above the current range [lo, hi]
  for (bool first = true;; first = false) {
    const uint64_t span = hi - lo;
    const int hb = span ? 63 - __clzll((long long)span) : 0;
    constexpr int kBinBits = kBins == 1024 ? 10 : (kBins == 512 ? 9 : 8);
    static_assert((1 << kBinBits) == kBins, "power-of-two bins");
    const int shift = hb > kBinBits - 1 ? hb - (kBinBits - 1) : 0;  // span >> shift < kBins
    if (!first) {
      for (int i = tid; i < kBins; i += NT) sh.hist[i] = 0;
      lds_sync();
    }
    visit([&](uint64_t x) __attribute__((always_inline)) {
      if (x >= lo && x <= hi) atomicAdd(&sh.hist[(uint32_t)((x - lo) >> shift)], 1u);
    });
    lds_sync();
    const uint32_t need_here = need - above;
    // thread t owns the upper bin kBins-1-2t and the lower bin kBins-2-2t,
    // so "bins above" is a prefix over threads
    const uint32_t bu = kBins - 1 - 2 * tid;
    const uint32_t h1 = sh.hist[bu], h0 = sh.hist[bu - 1];
    const uint32_t s = h0 + h1;
    const uint32_t incl = wave_scan_u32(s, 0u, uadd);
    if (lane == 63) sh.red_n[wave] = incl;
    lds_sync();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += sh.red_n[w];
    const uint32_t X = incl - s + before;  // keys in bins above bu
    if (X < need_here && need_here <= X + h1) {
      sh.bin = bu; sh.ca = X; sh.cb = h1;
    } else if (X + h1 < need_here && need_here <= X + s) {
      sh.bin = bu - 1; sh.ca = X + h1; sh.cb = h0;
    }
    lds_sync();
    const uint32_t b = sh.bin, ca = sh.ca, cb = sh.cb;
    const uint64_t gb = lo + ((uint64_t)b << shift);
    // (uniform; after the return nothing writes bin, ca, cb or the
    // histogram before another barrier)
    if (above + ca + cb <= target || shift == 0) return gb;
    lds_sync();  // every thread has read bin, ca, cb
    above += ca;
    const uint64_t top = gb + ((1ull << shift) - 1);
    lo = gb;
    hi = top < hi ? top : hi;
  }
}

}  // namespace csa
