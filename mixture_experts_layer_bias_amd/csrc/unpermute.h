// Per-element combine of the unpermute step, shared by the unpermute-reduce
// kernel and the fused decode launch.  forward_prefill.rs page,
// moe_unpermute_reduce_indexed (top-K-weighted sum of the token's expert rows)
// and the shared blend (weight 1 without a shared_expert_gate); forward.rs
// page, MoeLayer::apply_zero_expert (out[t,:] += zero_accum[t] * x[t,:]).
// Everything is summed in fp32 in one order (slots, then the identity experts'
// x term, then the shared expert) and rounded once to bf16.
#pragma once

#include "common.h"

namespace moe {

// acc[0..7] += wv * the 8 bf16 values of v
__device__ __forceinline__ void acc_bf16x8(float (&acc)[8], float wv, const u32x4& v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[2 * j] += wv * bf16_to_f32(v[j] & 0xFFFFu);
    acc[2 * j + 1] += wv * bf16_to_f32(v[j] >> 16);
  }
}

// the identity experts' term (summed weight `zero` times x), then the shared expert's output
__device__ __forceinline__ u32x4 finish_bf16x8(float (&acc)[8], float zero, const u32x4& xv, bool shared,
                                               const u32x4& sv) {
  if (zero != 0.f) acc_bf16x8(acc, zero, xv);
  if (shared) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16_to_f32(sv[j] & 0xFFFFu);
      acc[2 * j + 1] += bf16_to_f32(sv[j] >> 16);
    }
  }
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
  return o;
}

}  // namespace moe
