// Unpermute with the top-K-weighted reduce and the identity-expert and
// shared-expert blends, for gfx950.  forward_prefill.rs page,
// moe_unpermute_reduce_indexed and the shared blend (weight 1 without a
// shared_expert_gate); forward.rs page, MoeLayer::apply_zero_expert
// (out[t,:] += zero_accum[t] * x[t,:]).  One fp32 sum per element, rounded
// once to bf16.
#include "common.h"
#include "kernels.h"
#include "unpermute.h"

namespace moe {

// One block per token; threads stride over 8-column (16-byte) chunks of H.  A
// thread issues the loads of all K slot rows (and of x and the shared output)
// of a chunk before its first add, so a chunk costs one memory round trip; the
// adds then run in slot order.  KB >= K.
template <int KB>
__global__ __launch_bounds__(256) void k_unpermute_reduce(const uint16_t* __restrict__ y,
                                                          const int32_t* __restrict__ inv_perm,
                                                          const int32_t* __restrict__ ids,
                                                          const float* __restrict__ w,
                                                          const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ shared_y,
                                                          uint16_t* __restrict__ out, int H, int K, int E) {
  __shared__ int rows[KB];
  __shared__ float wk[KB];
  const int t = blockIdx.x;
  if (threadIdx.x < K) {
    const int id = ids[(size_t)t * K + threadIdx.x];
    rows[threadIdx.x] = id < E ? inv_perm[(size_t)t * K + threadIdx.x] : -1;
    wk[threadIdx.x] = w[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  float zero = 0.f;  // the identity experts' summed weight, added in slot order
  for (int k = 0; k < K; ++k)
    if (rows[k] < 0) zero += wk[k];
  const size_t xrow = (size_t)t * H;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    u32x4 v[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int r = k < K ? rows[k] : -1;
      v[k] = r >= 0 ? ld16(y + (size_t)r * H + c) : z4;
    }
    const u32x4 xv = zero != 0.f ? ld16(x + xrow + c) : z4;
    const u32x4 sv = shared_y ? ld16(shared_y + xrow + c) : z4;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KB; ++k)
      if (k < K && rows[k] >= 0) acc_bf16x8(acc, wk[k], v[k]);
    const u32x4 o = finish_bf16x8(acc, zero, xv, shared_y != nullptr, sv);
    st16(out + xrow + c, o);
  }
}

hipError_t launch_unpermute_reduce(const uint16_t* y_sorted, const int32_t* inv_perm, const int32_t* ids,
                                   const float* w, const uint16_t* x, const uint16_t* shared_y, uint16_t* out, int N,
                                   int H, int K, int E, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (K <= 8) k_unpermute_reduce<8><<<N, 256, 0, s>>>(y_sorted, inv_perm, ids, w, x, shared_y, out, H, K, E);
  else if (K <= 16) k_unpermute_reduce<16><<<N, 256, 0, s>>>(y_sorted, inv_perm, ids, w, x, shared_y, out, H, K, E);
  else k_unpermute_reduce<32><<<N, 256, 0, s>>>(y_sorted, inv_perm, ids, w, x, shared_y, out, H, K, E);
  return hipGetLastError();
}

}  // namespace moe
