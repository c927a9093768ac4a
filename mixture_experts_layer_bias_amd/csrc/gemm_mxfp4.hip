// Grouped expert GEMMs on MXFP4 weights (OCP Microscaling: FP4 E2M1 codes, one E8M0
// power-of-two scale per row and 32 consecutive K columns) with e4m3 activations, for gfx950.
//
// Same data flow as the bf16 and fp8 kernels (forward_prefill.rs page,
// run_routed_grouped_gemm; the forward.rs page's MXFP4 / E8M0 expert arm names
// the weight format).  The weights' block scales are exactly what the scaled
// MFMA consumes: v_mfma_scale_f32_32x32x64_f8f6f4 with A = e4m3 activations
// (scale 2^0) and B = E2M1 weights (lane l's 32 K values carry the E8M0 scale
// of its weight row and 32-column block), so a 128-column K step is two MFMAs
// whose sums start from zero; the step's result is promoted into the fp32
// accumulator with the activation row's fp32 scale on the vector ALU.
//
// Block tile BM = 128 rows x BN = 128 output columns, K step 128 columns
// (128 bytes of A, 64 bytes of packed B per row), 4 waves in 2 x 2, each wave
// 64 x 64 (x2 for gate and up).  Operands are staged through LDS with register
// prefetch of the next K step.  The gate/up epilogue computes h = silu(g) * u and
// quantises it per row over the tile's 128 columns to e4m3 (the recipe of
// moe_quantize_fp8); the down stage writes bf16.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int A_STRIDE = BK + 16;      // bytes per LDS row of A (e4m3)
constexpr int B_STRIDE = BK / 2 + 16;  // bytes per LDS row of B (two E2M1 codes per byte)
constexpr int E8M0_ONE = 127;          // E8M0 code of 2^0

template <int STAGE>
struct MxTile {
  static constexpr int BROWS = STAGE == 0 ? 2 * BN : BN;   // weight rows per tile
  static constexpr int A_LOADS = BM * (BK / 16) / 256;     // 16-byte chunks per thread
  static constexpr int B_LOADS = BROWS * (BK / 32) / 256;  // 64 bytes per row = four 16-byte chunks
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Operand order of this MFMA (e4m3 A, E2M1 B), measured on the device: a B lane (row l % 32,
// half h = l / 32) holds 32 E2M1 values whose scale is that lane's E8M0 byte, and its value e
// meets A position 32 (e / 16) + 16 h + e % 16, where A position q is byte q % 32 of the A lane of
// half q / 32.  So B lanes load their 32 consecutive K values (memory block h of the 64-wide step,
// one E8M0 code), and A lanes of half h load memory K 16 h .. 16 h + 15 into bytes 0..15 and
// memory K 32 + 16 h .. 32 + 16 h + 15 into bytes 16..31: every A byte then meets the B value of
// the same K.
__device__ __forceinline__ f32x16 mfma_e4m3_x_e2m1(i32x8 a, i32x8 b, int b_scale, f32x16 c) {
  // cbsz 0: A is e4m3; blgp 4: B is E2M1 (its first four registers hold the lane's 32 codes)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, 0, E8M0_ONE, 0, b_scale);
}

template <int STAGE>
__global__ __launch_bounds__(256, STAGE == 0 ? 1 : 2) void k_grouped_gemm_mxfp4(GroupedGemmArgs g) {
  using T = MxTile<STAGE>;
  __shared__ __align__(16) uint8_t a_lds[BM * A_STRIDE];
  __shared__ __align__(16) uint8_t b_lds[T::BROWS * B_STRIDE];
  __shared__ uint32_t s_bsc[T::BROWS];  // the four E8M0 codes of each weight row in this K step
  __shared__ float s_asc[BM];           // activation row scales of this K step
  __shared__ float s_amax[2][BM];       // gate/up epilogue: per-row amax of each column half
  __shared__ int s_prefix[kMaxGroups + 1];
  __shared__ int s_wsum[4];

  const int KD = STAGE == 0 ? g.H : g.I;
  const int NCOLS = STAGE == 0 ? g.I : g.H;
  const int NT = NCOLS / BN;
  const int KB = KD / BK;
  const TileCoord tc =
      schedule_tile(g.offsets, g.shared ? 1 : g.E, g.shared ? g.N : -1, BM, NT, s_prefix, s_wsum);
  if (tc.expert < 0) return;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int n0 = tc.n_tile * BN;

  const uint8_t *wa, *wb = nullptr;  // packed codes [rows, KD/2]
  const uint8_t *sa_w, *sb_w = nullptr;  // E8M0 codes [rows, KD/32]
  if (STAGE == 0) {
    wa = static_cast<const uint8_t*>(g.shared ? g.sh_gate : g.w_gate[tc.expert]);
    wb = static_cast<const uint8_t*>(g.shared ? g.sh_up : g.w_up[tc.expert]);
    sa_w = reinterpret_cast<const uint8_t*>(g.shared ? g.sh_gate_s : g.s_gate[tc.expert]);
    sb_w = reinterpret_cast<const uint8_t*>(g.shared ? g.sh_up_s : g.s_up[tc.expert]);
  } else {
    wa = static_cast<const uint8_t*>(g.shared ? g.sh_down : g.w_down[tc.expert]);
    sa_w = reinterpret_cast<const uint8_t*>(g.shared ? g.sh_down_s : g.s_down[tc.expert]);
  }

  // A: row tid / 8 (+ 32 i), 16-byte chunk tid % 8
  const uint8_t* a_src = static_cast<const uint8_t*>(g.a);
  const int lrow = tid >> 3, lcol = (tid & 7) * 16;
  const uint8_t* a_ptr[T::A_LOADS];
#pragma unroll
  for (int i = 0; i < T::A_LOADS; ++i) {
    int p = tc.row0 + lrow + 32 * i;
    if (p >= tc.row_end) p = tc.row_end - 1;  // rows past the segment are computed, never stored
    const long arow = STAGE == 0 ? (g.shared ? p : g.sorted_ids[p] / g.K) : p;
    a_ptr[i] = a_src + (size_t)arow * KD + lcol;
  }
  const float* asc_ptr = nullptr;  // threads 0..127: the scale row of A row tid
  if (tid < BM) {
    int p = tc.row0 + tid;
    if (p >= tc.row_end) p = tc.row_end - 1;
    const long arow = STAGE == 0 ? (g.shared ? p : g.sorted_ids[p] / g.K) : p;
    asc_ptr = g.a_scales + (size_t)arow * KB;
  }
  // B: weight row tid / 4 (+ 64 i), 16-byte chunk tid % 4 (gate/up: rows [0, BN) gate, then up)
  const int brow = tid >> 2, bcol = (tid & 3) * 16;
  auto weight_row = [&](int r, const uint8_t* base_a, const uint8_t* base_b, size_t row_bytes) {
    if (STAGE == 0) return r < BN ? base_a + (size_t)(n0 + r) * row_bytes : base_b + (size_t)(n0 + r - BN) * row_bytes;
    return base_a + (size_t)(n0 + r) * row_bytes;
  };
  const uint8_t* b_ptr[T::B_LOADS];
#pragma unroll
  for (int i = 0; i < T::B_LOADS; ++i) b_ptr[i] = weight_row(brow + 64 * i, wa, wb, (size_t)KD / 2) + bcol;
  // threads 0..BROWS-1: the E8M0 row of weight row tid (4 codes per K step, one dword)
  const uint8_t* bsc_ptr = tid < T::BROWS ? weight_row(tid, sa_w, sb_w, (size_t)KD / 32) : nullptr;

  u32x4 ra[T::A_LOADS], rb[T::B_LOADS];
  float rsc = 0.f;
  uint32_t rbs = 0;
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) ra[i] = ldg16(a_ptr[i] + (size_t)kb * BK);
#pragma unroll
    for (int i = 0; i < T::B_LOADS; ++i) rb[i] = ldg16(b_ptr[i] + (size_t)kb * (BK / 2));
    if (tid < BM) rsc = ldg_f32(asc_ptr + kb);
    if (tid < T::BROWS) rbs = *reinterpret_cast<const uint32_t*>(bsc_ptr + (size_t)kb * (BK / 32));
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) st16(a_lds + (lrow + 32 * i) * A_STRIDE + lcol, ra[i]);
#pragma unroll
    for (int i = 0; i < T::B_LOADS; ++i) st16(b_lds + (brow + 64 * i) * B_STRIDE + bcol, rb[i]);
    if (tid < BM) s_asc[tid] = rsc;
    if (tid < T::BROWS) s_bsc[tid] = rbs;
  };

  constexpr int NB = STAGE == 0 ? 4 : 2;
  f32x16 acc[2][NB];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][nb][r] = 0.f;

  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 31, half = lane >> 5;  // the lane's row and half of a 64-wide MFMA step
  auto item_row = [&](int r) { return 8 * (r / 4) + 4 * (lane / 32) + (r % 4); };

  load_tile(0);
  store_tile();
  __syncthreads();
  for (int kb = 0; kb < KB; ++kb) {
    if (kb + 1 < KB) load_tile(kb + 1);
    f32x16 blk[2][NB];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) blk[mi][nb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 64) {
      i32x8 af[2], bfr[NB];
      int bsc[NB];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const uint8_t* p = a_lds + (wm * 64 + mi * 32 + frow) * A_STRIDE + kk + 16 * half;
        const u32x4 lo = ld16(p), hi = ld16(p + 32);
        af[mi] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        // stage 0: nb 0,1 -> gate rows, nb 2,3 -> up rows of the same columns
        const int wr = (STAGE == 0 && nb >= 2 ? BN : 0) + wn * 64 + (nb & 1) * 32 + frow;
        const u32x4 c = ld16(b_lds + wr * B_STRIDE + (kk + 32 * half) / 2);  // two codes per byte
        bfr[nb] = i32x8{(int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0, 0, 0};
        bsc[nb] = (int)((s_bsc[wr] >> (8 * (kk / 32 + half))) & 0xFFu);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) blk[mi][nb] = mfma_e4m3_x_e2m1(af[mi], bfr[nb], bsc[nb], blk[mi][nb]);
    }
    // promote this K step: acc += blk * (activation row scale); the weight scales are inside blk
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float rs = s_asc[wm * 64 + mi * 32 + item_row(r)];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mi][nb][r] += blk[mi][nb][r] * rs;
      }
    __syncthreads();
    if (kb + 1 < KB) {
      store_tile();
      __syncthreads();
    }
  }

  if (STAGE == 1) {
    uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tc.row0 + wm * 64 + mi * 32 + item_row(r);
        if (row >= tc.row_end) continue;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int col = n0 + wn * 64 + ni * 32 + (lane % 32);
          out[(size_t)row * NCOLS + col] = (uint16_t)f32_to_bf16(acc[mi][ni][r]);
        }
      }
    return;
  }

  // ---- gate/up epilogue: h = silu(g) * u, quantised per row over this tile's 128 columns
  float h[2][16][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float m = 0.f;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        h[mi][r][ni] = silu(acc[mi][ni][r]) * acc[mi][ni + 2][r];
        m = fmaxf(m, fabsf(h[mi][r][ni]));
      }
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));  // the row's 32 lanes
      if ((lane & 31) == 0) s_amax[wn][wm * 64 + mi * 32 + item_row(r)] = m;
    }
  __syncthreads();
  uint8_t* out = static_cast<uint8_t*>(g.out);
  const int groups = NCOLS / 128;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int trow = wm * 64 + mi * 32 + item_row(r);
      const int row = tc.row0 + trow;
      const float amax = fmaxf(s_amax[0][trow], s_amax[1][trow]);
      const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
      if (row < tc.row_end) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int col = n0 + wn * 64 + ni * 32 + (lane % 32);
          out[(size_t)row * NCOLS + col] = (uint8_t)f32_to_e4m3(h[mi][r][ni] * inv);
        }
        if (wn == 0 && (lane & 31) == 0) g.out_scales[(size_t)row * groups + tc.n_tile] = amax > 0.f ? amax / 448.0f : 1.0f;
      }
    }
}

}  // namespace

hipError_t launch_grouped_gemm_mxfp4(const GroupedGemmArgs& g, hipStream_t s) {
  const int groups = g.shared ? 1 : g.E;
  const int rows = g.shared ? g.N : g.P;
  if (rows == 0) return hipSuccess;
  if (g.stage == 0) {
    k_grouped_gemm_mxfp4<0><<<grouped_grid(rows, groups, BM, g.I / BN), 256, 0, s>>>(g);
  } else {
    k_grouped_gemm_mxfp4<1><<<grouped_grid(rows, groups, BM, g.H / BN), 256, 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace moe
