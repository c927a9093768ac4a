/*
 * Seeded synthetic inputs for the MoE layer forward: one definition, compiled
 * for the host (gcc, OpenMP) and for gfx950 (hipcc), so that a tensor filled on
 * the GPU is bit-identical to the same tensor filled on the CPU.
 *
 * This file holds input synthesis only, none of the MoE method's arithmetic.
 *
 * Definition
 * ----------
 * key(seed, tag, sub)   = mix64(mix64(seed + GOLDEN*(tag+1)) ^ (sub * MUL_SUB))
 * word(key, c)          = mix64(key + GOLDEN*(c+1))              (64 random bits)
 * normal(key, i)        = (S - 393210) * 2^-16, where S is the sum of the twelve
 *                         16-bit fields of word(key, 3i), word(key, 3i+1),
 *                         word(key, 3i+2)  (Irwin-Hall sum of 12 uniforms:
 *                         mean 0, variance (2^32-1)/2^32, support +-6).
 *   Every step is integer arithmetic, and (S - 393210) fits in 20 bits, so the
 *   fp32 value is exact on every device.
 * value(key, i, sigma)  = fp32(normal(key, i) * sigma)  (one correctly rounded
 *                         fp32 multiply, identical on every IEEE device)
 * bf16 tensors          = round-to-nearest-even of value() to bfloat16
 * e4m3 tensors          = per 128x128 block of value(): S = fp32(amax / 448),
 *                         code = e4m3fn_rne_satfinite(fp32(v / S)); a zero block
 *                         has S = 1.  (OCP FP8 E4M3: bias 7, max 448, no inf.)
 * mxfp4 tensors         = per row, per 32 consecutive columns of value() (the OCP
 *                         Microscaling Formats v1.0 recipe for MXFP4): shared
 *                         exponent X = floor(log2(amax)) - 2 (2 = the largest
 *                         E2M1 exponent), scale code = X + 127 (E8M0), element
 *                         code = e2m1_rne_sat(v * 2^-X) (OCP FP4 E2M1: values
 *                         0, 0.5, 1, 1.5, 2, 3, 4, 6; beyond 6 saturates); a
 *                         zero block gets scale code 127 and zero codes.
 *                         Two codes per byte, the even column in the low nibble.
 * mix64 is the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014).
 */
#ifndef MOE_INPUTS_GEN_CORE_H
#define MOE_INPUTS_GEN_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define MI_FN __host__ __device__ static inline
#else
#define MI_FN static inline
#endif

#define MI_GOLDEN 0x9E3779B97F4A7C15ULL
#define MI_MUL_SUB 0xD1B54A32D192ED03ULL

/* tensor tags */
enum {
  MI_TAG_X = 1,
  MI_TAG_ROUTER = 2,
  MI_TAG_BIAS = 3,
  MI_TAG_GATE = 4,
  MI_TAG_UP = 5,
  MI_TAG_DOWN = 6,
  MI_TAG_SH_GATE = 7,
  MI_TAG_SH_UP = 8,
  MI_TAG_SH_DOWN = 9,
  MI_TAG_PERM = 10
};

MI_FN uint64_t mi_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

MI_FN uint64_t mi_key(uint64_t seed, uint32_t tag, uint32_t sub) {
  return mi_mix64(mi_mix64(seed + MI_GOLDEN * (uint64_t)(tag + 1)) ^ ((uint64_t)sub * MI_MUL_SUB));
}

MI_FN uint64_t mi_word(uint64_t key, uint64_t c) { return mi_mix64(key + MI_GOLDEN * (c + 1)); }

MI_FN int32_t mi_fields16(uint64_t w) {
  return (int32_t)(w & 0xFFFF) + (int32_t)((w >> 16) & 0xFFFF) + (int32_t)((w >> 32) & 0xFFFF) +
         (int32_t)(w >> 48);
}

MI_FN float mi_normal(uint64_t key, uint64_t i) {
  int32_t s = mi_fields16(mi_word(key, 3 * i)) + mi_fields16(mi_word(key, 3 * i + 1)) +
              mi_fields16(mi_word(key, 3 * i + 2)) - 393210;
  return (float)s * (1.0f / 65536.0f);
}

MI_FN float mi_value(uint64_t key, uint64_t i, float sigma) { return mi_normal(key, i) * sigma; }

MI_FN uint32_t mi_f32_bits(float f) {
  union {
    float f;
    uint32_t u;
  } c;
  c.f = f;
  return c.u;
}

MI_FN float mi_bits_f32(uint32_t u) {
  union {
    float f;
    uint32_t u;
  } c;
  c.u = u;
  return c.f;
}

/* fp32 -> bf16, round to nearest even (values here are always finite) */
MI_FN uint16_t mi_bf16_rne(float f) {
  uint32_t u = mi_f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* fp32 -> OCP e4m3fn, round to nearest even, saturate finite values to +-448 */
MI_FN uint8_t mi_e4m3_rne_sat(float f) {
  uint32_t u = mi_f32_bits(f);
  uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return (uint8_t)(sign | 0x7F); /* NaN */
  if (a >= 0x43E00000u) return (uint8_t)(sign | 0x7E); /* >= 448 (and inf) saturate */
  if (a < 0x3C800000u) {                               /* below 2^-6: subnormal step 2^-9 */
    float t = mi_bits_f32(a) * 512.0f;                /* exact power-of-two scaling */
    uint32_t n = (uint32_t)t;                         /* truncation */
    float frac = t - (float)n;                        /* exact */
    if (frac > 0.5f || (frac == 0.5f && (n & 1u))) n += 1u;
    return (uint8_t)(sign | n); /* n == 8 is the smallest normal, code 0x08 */
  }
  /* normal: keep 3 mantissa bits, round to nearest even on the dropped 20 */
  uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  r >>= 20;                                  /* (exp8 << 3) | mant3 in fp32 bias */
  uint32_t code = r - ((127u - 7u) << 3);    /* rebias 127 -> 7 */
  if (code > 0x7Eu) code = 0x7Eu;
  return (uint8_t)(sign | code);
}

/* fp32 -> OCP FP4 E2M1 code (sign in bit 3), round to nearest with ties to the even code,
 * finite values beyond 6 saturate to 6.  The magnitude codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6,
 * so each threshold below is the midpoint of two neighbours, assigned to the even code. */
MI_FN uint8_t mi_e2m1_rne_sat(float f) {
  uint8_t sign = (uint8_t)((mi_f32_bits(f) >> 28) & 0x8u);
  float a = f < 0.0f ? -f : f;
  uint8_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return (uint8_t)(sign | c);
}

/* E8M0 scale code of a 32-element block with maximum magnitude amax (a normal fp32 value or 0) */
MI_FN uint8_t mi_mx_scale_code(float amax) {
  if (!(amax > 0.0f)) return 127u;
  int e = (int)((mi_f32_bits(amax) >> 23) & 0xFFu) - 127; /* floor(log2(amax)) */
  int code = e - 2 + 127;
  return (uint8_t)(code < 0 ? 0 : (code > 254 ? 254 : code));
}

/* 2^-(code - 127) as fp32 (exact for the codes that occur here) */
MI_FN float mi_mx_inv_scale(uint8_t code) { return mi_bits_f32((uint32_t)(254 - code) << 23); }

#endif
