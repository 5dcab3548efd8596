// csa_select.hip -- exact top-k of a score array (csa_topk).
//
// Selection order (DS4X page, "CSA score/top-512 fusion"): larger score
// first, equal scores by lower row index.  Every row gets the 64-bit key
// (ord(score) << 32) | (2^32 - 1 - row), so the order is a plain unsigned
// comparison and all keys are distinct.  One workgroup per session finds the
// k-th largest key by an MSB-first radix select (8-bit digits, streaming the
// scores from memory, stopping as soon as the keys sharing the current
// prefix are exactly the ones still needed), gathers the keys at or above it
// and sorts them with a bitonic network in LDS.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kSelThreads = 1024;

struct SelectArgs {
  SelectSession s[CSA_MAX_SESSIONS];
  int k;
};

// Suffix-sum search over a 256-bin histogram by one wave: returns the digit d
// such that sum(h[d+1..255]) < need <= sum(h[d..255]); *above = sum(h[d+1..]).
__device__ int find_digit(const uint32_t *h, uint32_t need, uint32_t *above) {
  const int lane = threadIdx.x & 63;
  // lane owns bins 4*lane .. 4*lane+3
  uint32_t c0 = h[4 * lane], c1 = h[4 * lane + 1], c2 = h[4 * lane + 2], c3 = h[4 * lane + 3];
  uint32_t mine = c0 + c1 + c2 + c3;
  // inclusive suffix sum over lanes (lane 63 holds the top bins)
  uint32_t suf = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t v = __shfl_down(suf, off, 64);
    if (lane + off < 64) suf += v;
  }
  const uint32_t after = suf - mine;  // bins above this lane's four
  int digit = -1;
  uint32_t ab = 0;
  if (after < need && need <= suf) {
    uint32_t acc = after;
    if (acc + c3 >= need) { digit = 4 * lane + 3; ab = acc; }
    else { acc += c3;
      if (acc + c2 >= need) { digit = 4 * lane + 2; ab = acc; }
      else { acc += c2;
        if (acc + c1 >= need) { digit = 4 * lane + 1; ab = acc; }
        else { acc += c1; digit = 4 * lane; ab = acc; } } }
  }
  const unsigned long long ball = __ballot(digit >= 0);
  const int src = ball ? (int)__ffsll(ball) - 1 : 0;
  *above = __shfl(ab, src, 64);
  return __shfl(digit, src, 64);
}

// Bitonic sort, descending, of n2 (power of two, <= 1024) keys in LDS.
__device__ void bitonic_desc(uint64_t *keys, int n2) {
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (n2 >> 1); t += blockDim.x) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool desc = ((lo & size) == 0);
        const uint64_t a = keys[lo], b = keys[hi];
        if ((a < b) == desc) { keys[lo] = b; keys[hi] = a; }
      }
      __syncthreads();
    }
  }
}

__global__ void __launch_bounds__(kSelThreads) select_topk_kernel(const SelectArgs a) {
  const SelectSession &S = a.s[blockIdx.x];
  const int64_t n = S.n_rows;
  const int k = a.k;
  const int k_eff = (int)((n < (int64_t)k) ? n : (int64_t)k);

  __shared__ uint32_t hist[256];
  __shared__ uint64_t buf[1024];
  __shared__ uint64_t s_prefix, s_mask;
  __shared__ uint32_t s_need, s_done, s_cnt;

  if (threadIdx.x == 0) { s_prefix = 0; s_mask = 0; s_need = (uint32_t)k_eff; s_done = (k_eff == 0); s_cnt = 0; }
  __syncthreads();

  for (int shift = 56; shift >= 0 && !s_done; shift -= 8) {
    for (int t = threadIdx.x; t < 256; t += blockDim.x) hist[t] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix, mask = s_mask;
    for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
      const uint64_t key = make_key(S.scores[j], (uint32_t)j);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      uint32_t above;
      const int d = find_digit(hist, s_need, &above);
      if (threadIdx.x == 0) {
        const uint32_t need = s_need - above;
        s_prefix = prefix | ((uint64_t)d << shift);
        s_mask = mask | ((uint64_t)255u << shift);
        s_need = need;
        if (hist[d] == need) s_done = 1;
      }
    }
    __syncthreads();
  }

  // Keys >= threshold: exactly k_eff of them.
  const uint64_t thr = s_prefix;
  for (int t = threadIdx.x; t < 1024; t += blockDim.x) buf[t] = 0;
  __syncthreads();
  if (k_eff > 0) {
    for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
      const uint64_t key = make_key(S.scores[j], (uint32_t)j);
      if (key >= thr) {
        const uint32_t p = atomicAdd(&s_cnt, 1u);
        if (p < 1024u) buf[p] = key;
      }
    }
  }
  __syncthreads();
  int n2 = 1;
  while (n2 < k_eff) n2 <<= 1;
  if (n2 > 1) bitonic_desc(buf, n2);
  for (int t = threadIdx.x; t < k; t += blockDim.x) {
    if (t < k_eff) {
      const uint64_t key = buf[t];
      const uint32_t row = key_row(key);
      S.sel_idx[t] = (int32_t)row;
      if (S.sel_score) S.sel_score[t] = S.scores[row];
    } else {
      S.sel_idx[t] = -1;
      if (S.sel_score) S.sel_score[t] = -__builtin_inff();
    }
  }
}

hipError_t launch_select(const SelectSession *s, int n_sessions, int k, hipStream_t st) {
  SelectArgs a;
  for (int i = 0; i < n_sessions; ++i) a.s[i] = s[i];
  a.k = k;
  select_topk_kernel<<<n_sessions, kSelThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace csa
