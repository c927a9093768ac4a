// Per-token, per-128-column e4m3 quantisation of bf16 activations (the FP8
// expert path of the forward.rs and forward_batched.rs pages runs fp8 weight
// tables; the activations are quantised per token and per 128 columns).
//   amax = max |x| over the group; inv = 448 / amax (correctly rounded fp32);
//   code = e4m3_rne_satfinite(x * inv); scale = amax / 448; a zero group gets
//   scale 1 and zero codes.
#include "common.h"
#include "kernels.h"

namespace moe {

// One wave per 128-column group, two columns per lane.
__global__ __launch_bounds__(256) void k_quant_fp8(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq,
                                                   float* __restrict__ xs, int rows, int cols) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int groups_per_row = cols / 128;
  const long g = (long)blockIdx.x * 4 + wave;
  if (g >= (long)rows * groups_per_row) return;
  const long row = g / groups_per_row, grp = g % groups_per_row;
  const size_t off = (size_t)row * cols + (size_t)grp * 128 + lane * 2;
  const uint32_t two = *reinterpret_cast<const uint32_t*>(x + off);
  const float a = bf16_to_f32(two & 0xFFFFu), b = bf16_to_f32(two >> 16);
  const float amax = wave_max(fmaxf(fabsf(a), fabsf(b)));
  const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
  const uint32_t qa = f32_to_e4m3(a * inv), qb = f32_to_e4m3(b * inv);
  *reinterpret_cast<uint16_t*>(xq + off) = (uint16_t)(qa | (qb << 8));
  if (lane == 0) xs[(size_t)row * groups_per_row + grp] = sc;
}

hipError_t launch_quant_fp8(const uint16_t* x, uint8_t* xq, float* xs, int rows, int cols, hipStream_t s) {
  const long groups = (long)rows * (cols / 128);
  if (groups == 0) return hipSuccess;
  k_quant_fp8<<<(unsigned)((groups + 3) / 4), 256, 0, s>>>(x, xq, xs, rows, cols);
  return hipGetLastError();
}

}  // namespace moe
