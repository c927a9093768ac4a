// Unpermute with the top-K-weighted reduce and the identity-expert and
// shared-expert blends, for gfx950.  forward_prefill.rs page,
// moe_unpermute_reduce_indexed and the shared blend (output +=
// sigmoid(input . shared_expert_gate) * shared, weight 1 without that gate);
// forward.rs page, MoeLayer::apply_zero_expert (out[t,:] += zero_accum[t] *
// x[t,:]).  One fp32 sum per element, rounded once to bf16.
#include "common.h"
#include "kernels.h"
#include "unpermute.h"

namespace moe {

// One block per token; threads stride over 8-column (16-byte) chunks of H.  A
// thread issues the loads of all K slot rows (and of x and the shared output)
// of a chunk before its first add, so a chunk costs one memory round trip; the
// adds then run in slot order.  With a shared-expert gate, wave 0 first
// computes the token's shared weight.  KB >= K.
template <int KB>
__global__ __launch_bounds__(256) void k_unpermute_reduce(const uint16_t* __restrict__ y, ReduceArgs r) {
  __shared__ int rows[KB];
  __shared__ float wk[KB];
  __shared__ float s_shared_w;
  const int t = blockIdx.x, H = r.H, K = r.K;
  if (threadIdx.x < K) {
    const int id = r.ids[(size_t)t * K + threadIdx.x];
    rows[threadIdx.x] = id < r.E ? r.inv_perm[(size_t)t * K + threadIdx.x] : -1;
    wk[threadIdx.x] = r.w[(size_t)t * K + threadIdx.x];
  }
  const bool gated = r.shared_y && r.shared_gate;
  if (gated && threadIdx.x < kWave) {
    const float g = shared_gate_weight(r.x + (size_t)t * H, r.shared_gate, H);
    if (threadIdx.x == 0) s_shared_w = g;
  }
  __syncthreads();
  const float shared_w = gated ? s_shared_w : 1.0f;
  float zero = 0.f;  // the identity experts' summed weight, added in slot order
  for (int k = 0; k < K; ++k)
    if (rows[k] < 0) zero += wk[k];
  const size_t xrow = (size_t)t * H;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    u32x4 v[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int rr = k < K ? rows[k] : -1;
      v[k] = rr >= 0 ? ld16(y + (size_t)rr * H + c) : z4;
    }
    const u32x4 xv = zero != 0.f ? ld16(r.x + xrow + c) : z4;
    const u32x4 sv = r.shared_y ? ld16(r.shared_y + xrow + c) : z4;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KB; ++k)
      if (k < K && rows[k] >= 0) acc_bf16x8(acc, wk[k], v[k]);
    st16(r.out + xrow + c, finish_bf16x8(acc, zero, xv, r.shared_y != nullptr, sv, shared_w));
  }
}

hipError_t launch_unpermute_reduce(const uint16_t* y_sorted, const ReduceArgs& r, hipStream_t s) {
  if (r.N == 0) return hipSuccess;
  if (r.K <= 8) k_unpermute_reduce<8><<<r.N, 256, 0, s>>>(y_sorted, r);
  else if (r.K <= 16) k_unpermute_reduce<16><<<r.N, 256, 0, s>>>(y_sorted, r);
  else k_unpermute_reduce<32><<<r.N, 256, 0, s>>>(y_sorted, r);
  return hipGetLastError();
}

}  // namespace moe
