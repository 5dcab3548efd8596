// csa_decode.hip -- stand-alone row decoders (csa_dequant_idx /
// csa_dequant_kv): the element formats decoded in software, element by
// element (csa_device.hpp), into fp32 arrays.  The decode-step kernels do not
// call these: the scorer feeds the packed codes and scale bytes to the
// block-scaled matrix cores as they are stored, and the attention converts
// E4M3 codes with gfx950's fp8 conversion and applies the block scales as
// exact powers of two (csa_attn.hpp); that path is pinned bit for bit by the
// single-row attention tests.  csa_quantize_query's kernel is the
// quantizer the score kernel runs on its query fragments (csa_score.hpp).
#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "csa_score.hpp"

namespace csa {

// One thread per element; grid-stride over n_rows * 128.
__global__ void __launch_bounds__(256) dequant_idx_kernel(const uint8_t *__restrict__ rows, int64_t n,
                                                          float *__restrict__ out) {
  const int64_t total = n * 128;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = t >> 7;
    const int i = (int)(t & 127);
    const uint8_t *r = rows + j * kIdxRowBytes;
    const uint32_t code = (r[i >> 1] >> ((i & 1) * 4)) & 15u;
    out[t] = e2m1_value(code) * ue8m0_scale(r[64 + (i >> 5)]);
  }
}

__global__ void __launch_bounds__(256) dequant_kv_kernel(const uint8_t *__restrict__ rows, int64_t n,
                                                         float *__restrict__ out) {
  const int64_t total = n * 512;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = t >> 9;
    const int i = (int)(t & 511);
    const uint8_t *r = rows + j * kKvRowBytes;
    float v;
    if (i < kKvNope) {
      v = e4m3_value(r[i]) * ue8m0_scale(r[576 + (i >> 6)]);
    } else {
      const int o = kKvNope + 2 * (i - kKvNope);
      v = f16_value((uint32_t)r[o] | ((uint32_t)r[o + 1] << 8));
    }
    out[t] = v;
  }
}

// One thread per (head, 32-value block): the block quantized to MXFP4 and
// stored as the codes and scale byte of a 68-byte row.
__global__ void __launch_bounds__(256) quantize_query_kernel(const float *__restrict__ q, int n_heads,
                                                             uint8_t *__restrict__ rows) {
  const int t = threadIdx.x, h = t >> 2, b = t & 3;
  if (h >= n_heads) return;
  const float4 *src = reinterpret_cast<const float4 *>(q + (size_t)h * 128 + 32 * b);
  float x[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = src[i];
    x[4 * i] = v.x;
    x[4 * i + 1] = v.y;
    x[4 * i + 2] = v.z;
    x[4 * i + 3] = v.w;
  }
  QFrag<1> f;
  float deq[32];
  quantize_qfrag_fp4(f, x, deq);
  uint32_t *dst = reinterpret_cast<uint32_t *>(rows + (size_t)h * kIdxRowBytes + 16 * b);  // 4-byte aligned
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = (uint32_t)f.a[0][0][i];
  rows[(size_t)h * kIdxRowBytes + 64 + b] = (uint8_t)f.scw[0][0];
}

hipError_t launch_quantize_query(const float *q, int n_heads, uint8_t *rows, hipStream_t st) {
  quantize_query_kernel<<<1, 256, 0, st>>>(q, n_heads, rows);
  return hipGetLastError();
}

static unsigned grid_for(int64_t total) {
  int64_t b = (total + 255) / 256;
  if (b > 65536) b = 65536;
  return (unsigned)(b > 0 ? b : 1);
}

hipError_t launch_dequant_idx(const uint8_t *rows, int64_t n, float *out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  dequant_idx_kernel<<<grid_for(n * 128), 256, 0, st>>>(rows, n, out);
  return hipGetLastError();
}

hipError_t launch_dequant_kv(const uint8_t *rows, int64_t n, float *out, hipStream_t st) {
  if (n == 0) return hipSuccess;
  dequant_kv_kernel<<<grid_for(n * 512), 256, 0, st>>>(rows, n, out);
  return hipGetLastError();
}

}  // namespace csa
