// Unpermute with the top-K-weighted reduce and the identity-expert and
// shared-expert blends, for gfx950.  forward_prefill.rs page,
// moe_unpermute_reduce_indexed and the shared blend (weight 1 without a
// shared_expert_gate); forward.rs page, MoeLayer::apply_zero_expert
// (out[t,:] += zero_accum[t] * x[t,:]).  One fp32 sum per element, rounded
// once to bf16.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kMaxTopK = 32;

// One block per token; threads stride over 8-column (16-byte) chunks of H.
__global__ __launch_bounds__(256) void k_unpermute_reduce(const uint16_t* __restrict__ y,
                                                          const int32_t* __restrict__ inv_perm,
                                                          const int32_t* __restrict__ ids,
                                                          const float* __restrict__ w,
                                                          const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ shared_y,
                                                          uint16_t* __restrict__ out, int H, int K, int E) {
  __shared__ int rows[kMaxTopK];
  __shared__ float wk[kMaxTopK];
  __shared__ float zero_s;
  const int t = blockIdx.x;
  if (threadIdx.x < K) {
    const int id = ids[(size_t)t * K + threadIdx.x];
    const bool real = id < E;
    rows[threadIdx.x] = real ? inv_perm[(size_t)t * K + threadIdx.x] : -1;
    wk[threadIdx.x] = w[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float z = 0.f;
    for (int k = 0; k < K; ++k)
      if (rows[k] < 0) z += wk[k];
    zero_s = z;
  }
  __syncthreads();
  const float zero = zero_s;
  const size_t xrow = (size_t)t * H;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
      const int r = rows[k];
      if (r < 0) continue;
      const u32x4 v = ld16(y + (size_t)r * H + c);
      const float wv = wk[k];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += wv * bf16_to_f32(v[j] & 0xFFFFu);
        acc[2 * j + 1] += wv * bf16_to_f32(v[j] >> 16);
      }
    }
    if (zero != 0.f) {
      const u32x4 v = ld16(x + xrow + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += zero * bf16_to_f32(v[j] & 0xFFFFu);
        acc[2 * j + 1] += zero * bf16_to_f32(v[j] >> 16);
      }
    }
    if (shared_y) {
      const u32x4 v = ld16(shared_y + xrow + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += bf16_to_f32(v[j] & 0xFFFFu);
        acc[2 * j + 1] += bf16_to_f32(v[j] >> 16);
      }
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
    st16(out + xrow + c, o);
  }
}

hipError_t launch_unpermute_reduce(const uint16_t* y_sorted, const int32_t* inv_perm, const int32_t* ids,
                                   const float* w, const uint16_t* x, const uint16_t* shared_y, uint16_t* out, int N,
                                   int H, int K, int E, hipStream_t s) {
  if (N == 0) return hipSuccess;
  k_unpermute_reduce<<<N, 256, 0, s>>>(y_sorted, inv_perm, ids, w, x, shared_y, out, H, K, E);
  return hipGetLastError();
}

}  // namespace moe
