// csa_decode.hip -- stand-alone row decoders (csa_dequant_idx /
// csa_dequant_kv): the element formats decoded in software, element by
// element (csa_device.hpp), into fp32 arrays.  The decode-step kernels do not
// call these: the scorer feeds the packed codes and scale bytes to the
// block-scaled matrix cores as they are stored, and the attention converts
// E4M3 codes with gfx950's fp8 conversion and applies the block scales as
// exact powers of two (csa_attn.hpp); that path is pinned bit for bit by the
// single-row attention tests.
#include "csa_device.hpp"
#include "csa_internal.hpp"

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
