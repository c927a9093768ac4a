// Per-token, per-128-column e4m3 quantisation of bf16 activations (the FP8
// expert path of the forward.rs and forward_batched.rs pages runs fp8 weight
// tables; the activations are quantised per token and per 128 columns).
//   amax = max |x| over the group; inv = 448 / amax (correctly rounded fp32);
//   code = e4m3_rne_satfinite(x * inv); scale = amax / 448; a zero group gets
//   scale 1 and zero codes.
#include "common.h"
#include "kernels.h"

namespace moe {

// 16 lanes per 128-column group, 8 columns (one 16-byte load) per lane; each 16-lane row takes
// QG groups (all their loads issued before the first max), so a block covers 16 QG groups.  The
// group's amax is a max over rotations within the 16-lane DPP row, so every lane ends with it.
constexpr int QG = 1;

template <int ROT>
__device__ __forceinline__ float row_ror_max(float v) {
  return fmaxf(v, __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x120 + ROT, 0xF,
                                                                          0xF, false)));
}

__global__ __launch_bounds__(256) void k_quant_fp8(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq,
                                                   float* __restrict__ xs, int rows, int cols) {
  const int groups_per_row = cols / 128;
  const long ngroups = (long)rows * groups_per_row;
  const int sub = threadIdx.x % 16;
  const long g0 = ((long)blockIdx.x * 16 + threadIdx.x / 16) * QG;
  u32x4 v[QG];
  size_t off[QG];
#pragma unroll
  for (int q = 0; q < QG; ++q) {
    const long g = g0 + q < ngroups ? g0 + q : 0;  // the whole 16-lane row agrees
    off[q] = (size_t)(g / groups_per_row) * cols + (size_t)(g % groups_per_row) * 128 + sub * 8;
    v[q] = g0 + q < ngroups ? ldg16(x + off[q]) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int q = 0; q < QG; ++q) {
    float f[8], m = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_to_f32(v[q][i] & 0xFFFFu);
      f[2 * i + 1] = bf16_to_f32(v[q][i] >> 16);
      m = fmaxf(m, fmaxf(fabsf(f[2 * i]), fabsf(f[2 * i + 1])));
    }
    m = row_ror_max<8>(m);
    m = row_ror_max<4>(m);
    m = row_ror_max<2>(m);
    const float amax = row_ror_max<1>(m);
    const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= f32_to_e4m3(f[i] * inv) << (8 * i);
      hi |= f32_to_e4m3(f[4 + i] * inv) << (8 * i);
    }
    if (g0 + q < ngroups) {
      *reinterpret_cast<uint2*>(xq + off[q]) = make_uint2(lo, hi);
      if (sub == 0) xs[g0 + q] = amax > 0.f ? amax / 448.0f : 1.0f;  // [rows, groups_per_row] = group index
    }
  }
}

hipError_t launch_quant_fp8(const uint16_t* x, uint8_t* xq, float* xs, int rows, int cols, hipStream_t s) {
  const long groups = (long)rows * (cols / 128);
  if (groups == 0) return hipSuccess;
  k_quant_fp8<<<(unsigned)((groups + 16 * QG - 1) / (16 * QG)), 256, 0, s>>>(x, xq, xs, rows, cols);
  return hipGetLastError();
}

}  // namespace moe
