// gfx950 fill kernels for the seeded synthetic inputs defined in gen_core.h.
// Same definition as the host routines, so device and host fills are bit-identical.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gen_core.h"

__global__ void mi_k_fill_bf16(uint16_t* out, uint64_t n, uint64_t first, uint64_t key, float sigma) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    out[i] = mi_bf16_rne(mi_value(key, first + i, sigma));
}

__global__ void mi_k_fill_f32(float* out, uint64_t n, uint64_t first, uint64_t key, float sigma) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    out[i] = mi_value(key, first + i, sigma);
}

// One 256-thread block per 128x128 block of the matrix.
__global__ void __launch_bounds__(256) mi_k_fill_e4m3(uint8_t* q, float* scales, uint32_t rows, uint32_t cols,
                                                      uint64_t key, float sigma) {
  __shared__ float red[256];
  uint32_t bc = (cols + 127) / 128;
  uint32_t b = blockIdx.x;
  uint32_t r0 = (b / bc) * 128, c0 = (b % bc) * 128;
  uint32_t r1 = r0 + 128 < rows ? r0 + 128 : rows, c1 = c0 + 128 < cols ? c0 + 128 : cols;
  uint32_t w = c1 - c0, cnt = (r1 - r0) * w;
  float amax = 0.0f;
  for (uint32_t j = threadIdx.x; j < cnt; j += 256) {
    uint32_t r = r0 + j / w, c = c0 + j % w;
    float v = mi_value(key, (uint64_t)r * cols + c, sigma);
    amax = fmaxf(amax, fabsf(v));
  }
  red[threadIdx.x] = amax;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  amax = red[0];
  float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (threadIdx.x == 0) scales[b] = sc;
  for (uint32_t j = threadIdx.x; j < cnt; j += 256) {
    uint32_t r = r0 + j / w, c = c0 + j % w;
    q[(size_t)r * cols + c] = mi_e4m3_rne_sat(mi_value(key, (uint64_t)r * cols + c, sigma) / sc);
  }
}

// One thread per 32-element block of an MXFP4 matrix (same recipe as the host fill).
__global__ void __launch_bounds__(256) mi_k_fill_mxfp4(uint8_t* q, uint8_t* scales, uint64_t nb, uint64_t key,
                                                       float sigma) {
  for (uint64_t b = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += (uint64_t)gridDim.x * blockDim.x) {
    uint64_t e0 = b * 32;
    float v[32], amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
      v[j] = mi_value(key, e0 + (uint64_t)j, sigma);
      amax = fmaxf(amax, fabsf(v[j]));
    }
    uint8_t sc = mi_mx_scale_code(amax);
    float inv = mi_mx_inv_scale(sc);
    scales[b] = sc;
    for (int j = 0; j < 32; j += 2)
      q[e0 / 2 + (uint64_t)(j / 2)] =
          (uint8_t)(mi_e2m1_rne_sat(v[j] * inv) | (mi_e2m1_rne_sat(v[j + 1] * inv) << 4));
  }
}

static unsigned grid_for(uint64_t n) {
  uint64_t g = (n + 255) / 256;
  return (unsigned)(g > 65536 ? 65536 : (g == 0 ? 1 : g));
}

extern "C" int mi_dev_fill_bf16(void* out, uint64_t n, uint64_t first, uint64_t seed, uint32_t tag, uint32_t sub,
                                float sigma, hipStream_t stream) {
  if (n == 0) return 0;
  mi_k_fill_bf16<<<grid_for(n), 256, 0, stream>>>((uint16_t*)out, n, first, mi_key(seed, tag, sub), sigma);
  return (int)hipGetLastError();
}

extern "C" int mi_dev_fill_f32(void* out, uint64_t n, uint64_t first, uint64_t seed, uint32_t tag, uint32_t sub,
                               float sigma, hipStream_t stream) {
  if (n == 0) return 0;
  mi_k_fill_f32<<<grid_for(n), 256, 0, stream>>>((float*)out, n, first, mi_key(seed, tag, sub), sigma);
  return (int)hipGetLastError();
}

extern "C" int mi_dev_fill_mxfp4(void* q, void* scales, uint32_t rows, uint32_t cols, uint64_t seed, uint32_t tag,
                                 uint32_t sub, float sigma, hipStream_t stream) {
  uint64_t nb = (uint64_t)rows * (cols / 32);
  if (nb == 0) return 0;
  mi_k_fill_mxfp4<<<grid_for(nb), 256, 0, stream>>>((uint8_t*)q, (uint8_t*)scales, nb, mi_key(seed, tag, sub), sigma);
  return (int)hipGetLastError();
}

extern "C" int mi_dev_fill_e4m3(void* q, void* scales, uint32_t rows, uint32_t cols, uint64_t seed, uint32_t tag,
                                uint32_t sub, float sigma, hipStream_t stream) {
  if (rows == 0 || cols == 0) return 0;
  unsigned nb = ((rows + 127) / 128) * ((cols + 127) / 128);
  mi_k_fill_e4m3<<<nb, 256, 0, stream>>>((uint8_t*)q, (float*)scales, rows, cols, mi_key(seed, tag, sub), sigma);
  return (int)hipGetLastError();
}
