// Shared device helpers for the gfx950 MoE kernels: vector types, MFMA operand
// types, bf16 / e4m3 conversions and 64-wide wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) { return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16); }

// fp32 -> OCP e4m3 code, round to nearest even, finite values saturate at +-448.
// The value is split into a power-of-two binade and a significand in [8, 16)
// (three fraction bits), which v_rndne_f32 rounds; subnormals use the fixed
// step 2^-9.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fabsf(v);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {  // 2^-6: subnormal range
    code = (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8; 8 is the smallest normal (code 0x08)
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;  // -6..8
    float t = a * __uint_as_float((uint32_t)(127 + 3 - e) << 23);  // a * 2^(3-e), exact, in [8, 16)
    uint32_t m = (uint32_t)__builtin_rintf(t);                      // 8..16
    if (m == 16u) {
      m = 8u;
      e += 1;
    }
    code = ((uint32_t)(e + 7) << 3) | (m - 8u);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
    uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

// 16-byte load / store through a generic pointer (LDS or global, whichever the
// compiler can prove)
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// 16-byte load from GLOBAL memory.  Pointers read out of a device pointer table
// are generic to the compiler, which would emit flat loads; a flat load also
// counts against the LDS counter, so a wait for LDS reads would then wait for
// the in-flight prefetch from HBM as well.  The cast makes it a global load.
typedef const u32x4 __attribute__((address_space(1))) global_u32x4;
__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(global_u32x4*)(p); }
typedef const float __attribute__((address_space(1))) global_f32;
__device__ __forceinline__ float ldg_f32(const float* p) { return *(global_f32*)(p); }

__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

// e4m3 x e4m3 -> fp32, K = 64 per instruction (format code 0 = FP8 E4M3 for both operands;
// the block-scale operands are unused: E8M0 scale 1.0 is encoded as 127 but the
// unscaled form ignores them).
__device__ __forceinline__ f32x16 mfma_32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x128_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

}  // namespace moe
