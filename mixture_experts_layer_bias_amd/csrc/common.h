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

// Wave-wide reductions on DPP moves (no LDS round trips): an inclusive scan
// inside each 16-lane row with row_shr 1, 2, 4, 8, then row_bcast:15 and
// row_bcast:31 carry rows 0..2 into rows 1..3, so lane 63 holds the result,
// which readlane broadcasts.  Lanes a DPP move cannot source keep the identity.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t identity, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROW_MASK, 0xF, false);
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

__device__ __forceinline__ float wave_max(float v) {
  const uint32_t id = __float_as_uint(-INFINITY);
#define MOE_STEP(C, M) v = fmaxf(v, __uint_as_float(dpp_u32<C, M>(id, __float_as_uint(v))))
  MOE_STEP(kDppRowShr1, 0xF);
  MOE_STEP(kDppRowShr2, 0xF);
  MOE_STEP(kDppRowShr4, 0xF);
  MOE_STEP(kDppRowShr8, 0xF);
  MOE_STEP(kDppRowBcast15, 0xA);
  MOE_STEP(kDppRowBcast31, 0xC);
#undef MOE_STEP
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

// Sum in a fixed lane order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#define MOE_STEP(C, M) v = v + __uint_as_float(dpp_u32<C, M>(0u, __float_as_uint(v)))
  MOE_STEP(kDppRowShr1, 0xF);
  MOE_STEP(kDppRowShr2, 0xF);
  MOE_STEP(kDppRowShr4, 0xF);
  MOE_STEP(kDppRowShr8, 0xF);
  MOE_STEP(kDppRowBcast15, 0xA);
  MOE_STEP(kDppRowBcast31, 0xC);
#undef MOE_STEP
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#define MOE_STEP(C, M)                                                   \
  {                                                                      \
    const uint32_t lo = dpp_u32<C, M>(0u, (uint32_t)v);                  \
    const uint32_t hi = dpp_u32<C, M>(0u, (uint32_t)(v >> 32));          \
    const uint64_t o = ((uint64_t)hi << 32) | lo;                        \
    v = o > v ? o : v;                                                   \
  }
  MOE_STEP(kDppRowShr1, 0xF);
  MOE_STEP(kDppRowShr2, 0xF);
  MOE_STEP(kDppRowShr4, 0xF);
  MOE_STEP(kDppRowShr8, 0xF);
  MOE_STEP(kDppRowBcast15, 0xA);
  MOE_STEP(kDppRowBcast31, 0xC);
#undef MOE_STEP
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
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
