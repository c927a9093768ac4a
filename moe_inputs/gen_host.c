/* Host (CPU) fill routines for the seeded synthetic inputs defined in gen_core.h. */
#include <stddef.h>
#include <stdint.h>

#include "gen_core.h"

/* out[i] = bf16(value(key, first + i, sigma)), i < n */
void mi_host_fill_bf16(uint16_t* out, uint64_t n, uint64_t first, uint64_t seed, uint32_t tag,
                       uint32_t sub, float sigma) {
  uint64_t key = mi_key(seed, tag, sub);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = mi_bf16_rne(mi_value(key, first + (uint64_t)i, sigma));
}

/* out[i] = value(key, first + i, sigma) as fp32 */
void mi_host_fill_f32(float* out, uint64_t n, uint64_t first, uint64_t seed, uint32_t tag, uint32_t sub,
                      float sigma) {
  uint64_t key = mi_key(seed, tag, sub);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = mi_value(key, first + (uint64_t)i, sigma);
}

/* A [rows, cols] row-major matrix of value(key, r*cols + c, sigma) in MXFP4: q [rows, cols/2] packed
 * E2M1 codes (even column in the low nibble), scales [rows, cols/32] E8M0 codes.  cols % 32 == 0. */
void mi_host_fill_mxfp4(uint8_t* q, uint8_t* scales, uint32_t rows, uint32_t cols, uint64_t seed, uint32_t tag,
                        uint32_t sub, float sigma) {
  uint64_t key = mi_key(seed, tag, sub);
  uint64_t nb = (uint64_t)rows * (cols / 32);
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < (int64_t)nb; ++b) {
    uint64_t e0 = (uint64_t)b * 32; /* first element: blocks never straddle rows */
    float v[32], amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
      v[j] = mi_value(key, e0 + (uint64_t)j, sigma);
      float a = v[j] < 0 ? -v[j] : v[j];
      amax = a > amax ? a : amax;
    }
    uint8_t sc = mi_mx_scale_code(amax);
    float inv = mi_mx_inv_scale(sc);
    scales[b] = sc;
    for (int j = 0; j < 32; j += 2)
      q[e0 / 2 + (uint64_t)(j / 2)] =
          (uint8_t)(mi_e2m1_rne_sat(v[j] * inv) | (mi_e2m1_rne_sat(v[j + 1] * inv) << 4));
  }
}

/* A [rows, cols] row-major matrix of value(key, r*cols + c, sigma), stored as e4m3 codes
 * with one fp32 scale per 128x128 block: scales[(r/128) * ceil(cols/128) + c/128]. */
void mi_host_fill_e4m3(uint8_t* q, float* scales, uint32_t rows, uint32_t cols, uint64_t seed, uint32_t tag,
                       uint32_t sub, float sigma) {
  uint64_t key = mi_key(seed, tag, sub);
  uint32_t br = (rows + 127) / 128, bc = (cols + 127) / 128;
#pragma omp parallel for schedule(dynamic)
  for (int64_t b = 0; b < (int64_t)br * bc; ++b) {
    uint32_t r0 = (uint32_t)(b / bc) * 128, c0 = (uint32_t)(b % bc) * 128;
    uint32_t r1 = r0 + 128 < rows ? r0 + 128 : rows, c1 = c0 + 128 < cols ? c0 + 128 : cols;
    float amax = 0.0f;
    for (uint32_t r = r0; r < r1; ++r)
      for (uint32_t c = c0; c < c1; ++c) {
        float v = mi_value(key, (uint64_t)r * cols + c, sigma);
        float a = v < 0 ? -v : v;
        amax = a > amax ? a : amax;
      }
    float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    scales[b] = s;
    for (uint32_t r = r0; r < r1; ++r)
      for (uint32_t c = c0; c < c1; ++c)
        q[(size_t)r * cols + c] = mi_e4m3_rne_sat(mi_value(key, (uint64_t)r * cols + c, sigma) / s);
  }
}
