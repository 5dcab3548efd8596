// csa_pack.hip -- new rows in the packed formats and the merge of two
// attention results.
//
// Packing (DS4X page, "Packed cache ABI": compressed and raw-ring rows are
// stored as 583-byte KV rows, compressed indexer rows as 68-byte rows; the
// page names the formats, not the conversion): the OCP MX v1.0 block
// conversion.  Per block the UE8M0 byte is floor(log2 amax) - emax + 127
// (emax 8 for E4M3, 2 for E2M1) clamped to [0, 254], 127 for an all-zero
// block; each element v / 2^(byte-127) is rounded to the nearest element
// value, ties to the even significand, saturating (448, 6), and a value that
// rounds to zero is stored as +0.  RoPE values are IEEE binary16, round to
// nearest even.  pack_kernel: one workgroup of nine waves per row, waves
// 0..6 one E4M3 block each (a lane per element), wave 7 the 64 RoPE values,
// wave 8 the indexer row (16 lanes per 32-value block, two values a lane).
//
// Merge (the sliding-window ring and the compressed rows in one softmax):
// with a, b the two log-sum-exps and M = max(a, b),
//   out = (e^{a-M} out_a + e^{b-M} out_b) / (e^{a-M} + e^{b-M}),
//   lse = M + log(e^{a-M} + e^{b-M});
// a side with lse = -inf (no row) weighs nothing.  One thread per (head,
// dimension).
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kKvDim = CSA_KV_DIM;

// The UE8M0 byte of a block whose largest magnitude is amax (finite).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax, int emax) {
  if (amax == 0.0f) return 127u;
  const int ef = (int)(__float_as_uint(amax) >> 23);  // 0 for a subnormal amax: the byte clamps to 0
  const int b = ef == 0 ? 0 : ef - emax;               // floor(log2 amax) - emax + 127
  return (uint32_t)(b < 0 ? 0 : (b > 254 ? 254 : b));
}

// 2^(127 - byte) as fp32 (byte <= 254: 2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float inv_scale(uint32_t byte) {
  return byte == 254u ? __uint_as_float(0x00400000u) : __uint_as_float((254u - byte) << 23);
}

// E4M3 ("FN") code of y: round to nearest even, saturating at 448, a value
// that rounds to zero gives +0.
__device__ __forceinline__ uint32_t e4m3_round(float y) {
  const float a = fabsf(y);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0x1p-6f) {  // subnormal grid: multiples of 2^-9 (8 * 2^-9 is the smallest normal, code 8)
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    uint32_t bits = __float_as_uint(a);
    bits += 0x7FFFFu + ((bits >> 20) & 1u);  // round the fp32 significand to 3 bits, ties to even
    bits &= 0xFFF00000u;
    const float r = __uint_as_float(bits);
    if (r > 448.0f) {
      code = 0x7Eu;
    } else {
      const uint32_t e = (bits >> 23) - 127u + 7u;  // >= 1
      code = (e << 3) | ((bits >> 20) & 7u);
    }
  }
  return (code != 0u && y < 0.0f) ? (code | 0x80u) : code;
}

// E2M1 magnitude code of |y| (round to nearest even, saturating at 6; ties
// 0|0.5 -> 0, 0.5|1 -> 1, 1|1.5 -> 1, 1.5|2 -> 2, 2|3 -> 2, 3|4 -> 4, 4|6 -> 4),
// sign bit 3 for a negative nonzero result.
__device__ __forceinline__ uint32_t e2m1_pack_round(float y) {
  const float a = fabsf(y);
  const uint32_t c = (a > 0.25f ? 1u : 0u) + (a >= 0.75f ? 1u : 0u) + (a > 1.25f ? 1u : 0u) + (a >= 1.75f ? 1u : 0u) +
                     (a > 2.5f ? 1u : 0u) + (a >= 3.5f ? 1u : 0u) + (a > 5.0f ? 1u : 0u);
  return (c != 0u && y < 0.0f) ? (c | 8u) : c;
}

__device__ __forceinline__ float wave_max_abs(float x, int width) {
  float m = fabsf(x);
  for (int o = 1; o < width; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

constexpr int kPackThreads = 9 * 64;

__global__ void __launch_bounds__(kPackThreads) pack_kernel(const float *__restrict__ kv_vals,
                                                            const float *__restrict__ idx_vals, int64_t n,
                                                            uint8_t *__restrict__ kv_rows,
                                                            uint8_t *__restrict__ idx_rows) {
  const int64_t j = blockIdx.x;
  if (j >= n) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave < 7) {  // E4M3 block `wave`
    if (!kv_vals) return;
    const float x = kv_vals[j * kKvDim + 64 * wave + lane];
    const uint32_t byte = mx_scale_byte(wave_max_abs(x, 64), 8);
    uint8_t *r = kv_rows + j * kKvRowBytes;
    r[64 * wave + lane] = (uint8_t)e4m3_round(x * inv_scale(byte));
    if (lane == 0) r[576 + wave] = (uint8_t)byte;
  } else if (wave == 7) {  // the RoPE values
    if (!kv_vals) return;
    const float x = kv_vals[j * kKvDim + kKvNope + lane];
    const uint16_t h = __builtin_bit_cast(uint16_t, (_Float16)x);
    uint8_t *r = kv_rows + j * kKvRowBytes + kKvNope + 2 * lane;
    r[0] = (uint8_t)(h & 0xFFu);
    r[1] = (uint8_t)(h >> 8);
  } else {  // the indexer row: lane l holds values 2l, 2l + 1 (block l / 16)
    if (!idx_vals) return;
    const float2 x = *reinterpret_cast<const float2 *>(idx_vals + j * 128 + 2 * lane);
    float m = fmaxf(fabsf(x.x), fabsf(x.y));
    for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const uint32_t byte = mx_scale_byte(m, 2);
    const float inv = inv_scale(byte);
    const uint32_t c0 = e2m1_pack_round(x.x * inv), c1 = e2m1_pack_round(x.y * inv);
    uint8_t *r = idx_rows + j * kIdxRowBytes;
    r[lane] = (uint8_t)(c0 | (c1 << 4));
    if ((lane & 15) == 0) r[64 + (lane >> 4)] = (uint8_t)byte;
  }
}

hipError_t launch_pack(const float *kv_vals, const float *idx_vals, int64_t n, uint8_t *kv_rows, uint8_t *idx_rows,
                       hipStream_t st) {
  if (n == 0) return hipSuccess;
  pack_kernel<<<dim3((unsigned)n), kPackThreads, 0, st>>>(kv_vals, idx_vals, n, kv_rows, idx_rows);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) lse_merge_kernel(const float *out_a, const float *lse_a, const float *out_b,
                                                        const float *lse_b, int n_heads, float *out, float *lse) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n_heads * kKvDim) return;
  const int h = t / kKvDim;
  const float a = lse_a[h], b = lse_b[h];
  const float M = fmaxf(a, b);
  float o = 0.0f, l = -__builtin_inff();
  if (M != -__builtin_inff()) {
    const float wa = a == -__builtin_inff() ? 0.0f : __expf(a - M);
    const float wb = b == -__builtin_inff() ? 0.0f : __expf(b - M);
    const float xa = wa == 0.0f ? 0.0f : wa * out_a[t];
    const float xb = wb == 0.0f ? 0.0f : wb * out_b[t];
    o = (xa + xb) / (wa + wb);
    l = M + logf(wa + wb);
  }
  out[t] = o;
  if (lse && (t % kKvDim) == 0) lse[h] = l;
}

hipError_t launch_lse_merge(const float *out_a, const float *lse_a, const float *out_b, const float *lse_b,
                            int n_heads, float *out, float *lse, hipStream_t st) {
  const int total = n_heads * kKvDim;
  lse_merge_kernel<<<dim3((unsigned)((total + 255) / 256)), 256, 0, st>>>(out_a, lse_a, out_b, lse_b, n_heads, out, lse);
  return hipGetLastError();
}

}  // namespace csa
