// Router gate GEMM and top-K scoring for gfx950.
//
// Gate GEMM: forward_prefill.rs page (MoeLayer::forward_prefill, gate GEMM
// step) and forward_batched.rs page (the router width counts the
// zero-computation experts).  Scoring and selection: forward.rs page,
// MoeLayer::forward top-K arms (softmax; sigmoid + correction bias for
// selection, unbiased weights renormalised then scaled; softmax + correction
// bias with the zero-expert fold).
#include "common.h"
#include "kernels.h"

namespace moe {

// logits[N, R] = x[N, H] . router_w[R, H]^T on v_mfma_f32_16x16x32_bf16.
// A block of 4 waves covers MT*16 tokens x 64 router columns; each wave owns
// 16 columns and MT 16-row sub-tiles, so one B fragment feeds MT MFMAs.
// Operand fragments are loaded straight from global memory (16 B per lane):
// lane l holds row l%16 and the 8 consecutive k of chunk l/16 for both A and B,
// which is a consistent k assignment for the dot product.  The router is
// < 1% of the layer's work, so it does not stage through LDS.
template <int MT>
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ wr, float* __restrict__ logits,
                                                       int N, int H, int R) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int m0 = blockIdx.x * (16 * MT);
  const int ncol = blockIdx.y * 64 + wave * 16 + (lane % 16);
  const int kofs = (lane / 16) * 8;
  const bool nvalid = ncol < R;
  const uint16_t* bp = wr + (size_t)(nvalid ? ncol : 0) * H + kofs;
  const uint16_t* ap[MT];
  bool avalid[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int row = m0 + mt * 16 + (lane % 16);
    avalid[mt] = row < N;
    ap[mt] = x + (size_t)(avalid[mt] ? row : 0) * H + kofs;
  }
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int k = 0; k < H; k += 64) {
    u32x4 b0 = nvalid ? ld16(bp + k) : zero;
    u32x4 b1 = nvalid ? ld16(bp + k + 32) : zero;
    u32x4 a0[MT], a1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      a0[mt] = avalid[mt] ? ld16(ap[mt] + k) : zero;
      a1[mt] = avalid[mt] ? ld16(ap[mt] + k + 32) : zero;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] = mfma_16x16x32_bf16(a0[mt], b0, acc[mt]);
      acc[mt] = mfma_16x16x32_bf16(a1[mt], b1, acc[mt]);
    }
  }
  // D layout of the 16x16 MFMA: lane l, item r -> row 4*(l/16) + r, column l%16
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int row = m0 + mt * 16 + (lane / 16) * 4 + r;
      if (row < N && nvalid) logits[(size_t)row * R + ncol] = acc[mt][r];
    }
}

// One wave per token: scores in fp32, then K rounds of a wave-wide arg-max on
// a 64-bit key (order-preserving score bits, then the complement of the
// column), so ties go to the lower column and slots come out in descending
// order.  MAXJ = ceil(R/64) scores per lane.
__device__ __forceinline__ uint32_t order_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int MAXJ>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, const float* __restrict__ bias,
                                              int32_t* __restrict__ ids, float* __restrict__ w,
                                              float* __restrict__ zero_w, int N, int R, int E, int K, int scoring,
                                              int renorm, float scale) {
  __shared__ float p_lds[4][MAXJ * 64];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + wave;
  if (t >= N) return;  // the whole wave leaves; no block barrier below
  const float* lg = logits + (size_t)t * R;
  float p[MAXJ];
  if (scoring == 0) {
    float v[MAXJ];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      int r = lane + 64 * j;
      v[j] = r < R ? lg[r] : -INFINITY;
      m = fmaxf(m, v[j]);
    }
    m = wave_max(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      p[j] = (lane + 64 * j) < R ? expf(v[j] - m) : 0.f;
      s += p[j];
    }
    s = wave_sum(s);
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) p[j] = p[j] / s;
  } else {
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      int r = lane + 64 * j;
      p[j] = r < R ? 1.0f / (1.0f + expf(-lg[r])) : 0.f;
    }
  }
  float sel[MAXJ];
  uint32_t avail = 0;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    int r = lane + 64 * j;
    if (r < R) {
      p_lds[wave][r] = p[j];
      sel[j] = bias ? p[j] + bias[r] : p[j];
      avail |= 1u << j;
    } else {
      sel[j] = 0.f;
    }
  }
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      uint64_t key = ((uint64_t)order_bits(sel[j]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * j));
      if ((avail >> j) & 1u) best = key > best ? key : best;
    }
    best = wave_max_u64(best);
    const int r_star = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
#pragma unroll
    for (int j = 0; j < MAXJ; ++j)
      if (lane + 64 * j == r_star) avail &= ~(1u << j);
    if (lane == k) my_id = r_star;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float my_p = lane < K ? p_lds[wave][my_id] : 0.f;
  float wk = my_p;
  if (renorm) {
    float tot = wave_sum(my_p);
    wk = my_p / tot;
  }
  wk *= scale;
  float zsum = wave_sum((lane < K && my_id >= E) ? wk : 0.f);
  if (lane < K) {
    ids[(size_t)t * K + lane] = my_id;
    w[(size_t)t * K + lane] = wk;
  }
  if (lane == 0 && zero_w) zero_w[t] = zsum;
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* router_w, float* logits, int N, int H, int R,
                                hipStream_t s) {
  if (N == 0) return hipSuccess;
  dim3 block(256);
  if (N >= 256) {
    dim3 grid((N + 63) / 64, (R + 63) / 64);
    k_router_logits<4><<<grid, block, 0, s>>>(x, router_w, logits, N, H, R);
  } else {
    dim3 grid((N + 15) / 16, (R + 63) / 64);
    k_router_logits<1><<<grid, block, 0, s>>>(x, router_w, logits, N, H, R);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const float* bias, int32_t* ids, float* w, float* zero_w, int N, int R,
                       int E, int K, int scoring, int renormalize, float routed_scale, hipStream_t s) {
  if (N == 0) return hipSuccess;
  dim3 grid((N + 3) / 4), block(256);
  const int maxj = (R + 63) / 64;
#define MOE_TOPK_CASE(J)                                                                                 \
  case J:                                                                                                \
    k_topk<J><<<grid, block, 0, s>>>(logits, bias, ids, w, zero_w, N, R, E, K, scoring, renormalize,     \
                                     routed_scale);                                                      \
    break;
  switch (maxj) {
    MOE_TOPK_CASE(1)
    MOE_TOPK_CASE(2)
    MOE_TOPK_CASE(3)
    MOE_TOPK_CASE(4)
    MOE_TOPK_CASE(5)
    MOE_TOPK_CASE(6)
    MOE_TOPK_CASE(8)
    MOE_TOPK_CASE(16)
    default:
      if (maxj <= 8)
        k_topk<8><<<grid, block, 0, s>>>(logits, bias, ids, w, zero_w, N, R, E, K, scoring, renormalize,
                                         routed_scale);
      else
        k_topk<16><<<grid, block, 0, s>>>(logits, bias, ids, w, zero_w, N, R, E, K, scoring, renormalize,
                                          routed_scale);
  }
#undef MOE_TOPK_CASE
  return hipGetLastError();
}

}  // namespace moe
