// Per-element combine of the unpermute step, shared by the unpermute-reduce
// kernel and the fused decode launch.  forward_prefill.rs page,
// moe_unpermute_reduce_indexed (top-K-weighted sum of the token's expert rows)
// and the shared blend (output += sigmoid(input . shared_expert_gate) * shared,
// weight 1 without a shared_expert_gate); forward.rs page,
// MoeLayer::apply_zero_expert (out[t,:] += zero_accum[t] * x[t,:]).
// Everything is summed in fp32 in one order (slots, then the identity experts'
// x term, then the weighted shared expert) and rounded once to bf16.
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

// The shared expert's weight for one token, computed by the calling wave: sigmoid of the fp32
// dot product of the token's row with the gate row (lane l adds the products of 8-column chunks
// l, l + 64, ... in order, then the wave adds the lane sums).  Every lane gets the result.
__device__ __forceinline__ float shared_gate_weight(const uint16_t* xrow, const uint16_t* gate, int H) {
  float acc = 0.f;
  for (int c = (threadIdx.x % kWave) * 8; c < H; c += kWave * 8) {
    const u32x4 xv = ld16(xrow + c), gv = ld16(gate + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf(bf16_to_f32(xv[j] & 0xFFFFu), bf16_to_f32(gv[j] & 0xFFFFu), acc);
      acc = fmaf(bf16_to_f32(xv[j] >> 16), bf16_to_f32(gv[j] >> 16), acc);
    }
  }
  const float z = wave_sum(acc);
  return 1.0f / (1.0f + expf(-z));
}

// the identity experts' term (summed weight `zero` times x), then the shared expert's output
// times its weight `shared_w` (1 without a gate, which adds it unchanged)
__device__ __forceinline__ u32x4 finish_bf16x8(float (&acc)[8], float zero, const u32x4& xv, bool shared,
                                               const u32x4& sv, float shared_w) {
  if (zero != 0.f) acc_bf16x8(acc, zero, xv);
  if (shared) acc_bf16x8(acc, shared_w, sv);
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
  return o;
}

}  // namespace moe
