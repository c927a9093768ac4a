// Grouped expert GEMMs on bf16 weights for gfx950 (v_mfma_f32_32x32x16_bf16).
//
// forward_prefill.rs page, run_routed_grouped_gemm: a grouped gate/up GEMM,
// the activation and a grouped down GEMM over the rows sorted by expert; the
// shared expert is one more group holding every token (run_shared_expert_prefill).
//
// Block tile: BM = 128 sorted rows x BN = 128 output columns, K step BK = 64,
// 4 waves in a 2 x 2 arrangement, each wave 64 x 64 outputs as 2 x 2 MFMA
// 32x32 tiles.  The gate/up stage loads the gate AND the up rows of the same
// 128 columns (256 weight rows), keeps both accumulators in registers and
// applies silu(g) * u in the epilogue, so h is written once in bf16.  The A
// rows of the gate/up stage are gathered from x through sorted_ids / K.
// A and B tiles are staged through LDS with a 16-byte pad per row (row stride
// 144 B) against bank conflicts; the next K step's global loads are issued
// before the current step's MFMAs (register prefetch).
//
// STAGE 0: gate/up.  STAGE 1: down over 128 output columns.  STAGE 2: down over
// 256 output columns (H a multiple of 256), the same 256 weight rows, 4 MFMA
// column blocks per wave and registers as gate/up: a wave's 64 x 128 outputs
// read 0.75 LDS fragments per MFMA instead of 1.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row

template <int STAGE>
struct Bf16Tile {
  static constexpr int BROWS = STAGE == 1 ? BN : 2 * BN;  // weight rows per tile
  static constexpr int COLS = STAGE == 2 ? 2 * BN : BN;   // output columns per tile
  static constexpr int A_LOADS = BM * (BK / 8) / 256;      // 16-byte chunks per thread
  static constexpr int B_LOADS = BROWS * (BK / 8) / 256;
  static constexpr int LDS_BYTES = (BM + BROWS) * LDS_STRIDE * 2;
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <int STAGE>
__global__ __launch_bounds__(256, 2) void k_grouped_gemm_bf16(GroupedGemmArgs g) {
  using T = Bf16Tile<STAGE>;
  __shared__ __align__(16) uint16_t lds[T::LDS_BYTES / 2];
  uint16_t* a_lds = lds;
  uint16_t* b_lds = lds + BM * LDS_STRIDE;
  __shared__ int s_prefix[kMaxGroups + 1];
  __shared__ int s_wsum[4];

  const Groups G = gemm_groups(g, STAGE, T::COLS);
  const TileCoord tc = schedule_tile(G, BM, s_prefix, s_wsum);
  if (tc.expert < 0) return;
  const bool sh = tc.expert == G.nr;  // the shared expert's group
  const int KD = STAGE == 0 ? g.H : (sh ? g.Is : g.I);     // reduction length
  const int NCOLS = STAGE == 0 ? (sh ? g.Is : g.I) : g.H;  // output columns

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int n0 = tc.n_tile * T::COLS;

  // ---- operand pointers
  const uint16_t* wa;  // gate (stage 0) or down (stage 1) weights
  const uint16_t* wb = nullptr;  // up weights (stage 0)
  if (STAGE == 0) {
    wa = static_cast<const uint16_t*>(sh ? g.sh_gate : g.w_gate[tc.expert]);
    wb = static_cast<const uint16_t*>(sh ? g.sh_up : g.w_up[tc.expert]);
  } else {
    wa = static_cast<const uint16_t*>(sh ? g.sh_down : g.w_down[tc.expert]);
  }
  const uint16_t* a_src = static_cast<const uint16_t*>(sh ? g.sh_a : g.a);

  const int lrow = tid >> 3;       // 0..31: row within a 32-row slab of the tile
  const int lcol = (tid & 7) * 8;  // bf16 column of this thread's 16-byte chunk
  const uint16_t* a_ptr[T::A_LOADS];
#pragma unroll
  for (int i = 0; i < T::A_LOADS; ++i) {
    int p = tc.row0 + lrow + 32 * i;
    if (p >= tc.row_end) p = tc.row_end - 1;  // clamp: rows past the segment are computed, never stored
    long arow;
    if (STAGE == 0) arow = sh ? p : g.sorted_ids[p] / g.K;
    else arow = p;
    a_ptr[i] = a_src + (size_t)arow * KD + lcol;
  }
  const uint16_t* b_ptr[T::B_LOADS];
#pragma unroll
  for (int i = 0; i < T::B_LOADS; ++i) {
    const int r = lrow + 32 * i;  // 0..BROWS-1
    if (STAGE == 0) {
      b_ptr[i] = (r < BN ? wa + (size_t)(n0 + r) * KD : wb + (size_t)(n0 + r - BN) * KD) + lcol;
    } else {
      b_ptr[i] = wa + (size_t)(n0 + r) * KD + lcol;
    }
  }

  u32x4 ra[T::A_LOADS], rb[T::B_LOADS];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) ra[i] = ldg16(a_ptr[i] + k0);
#pragma unroll
    for (int i = 0; i < T::B_LOADS; ++i) rb[i] = ldg16(b_ptr[i] + k0);
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) st16(a_lds + (lrow + 32 * i) * LDS_STRIDE + lcol, ra[i]);
#pragma unroll
    for (int i = 0; i < T::B_LOADS; ++i) st16(b_lds + (lrow + 32 * i) * LDS_STRIDE + lcol, rb[i]);
  };

  constexpr int NB = STAGE == 1 ? 2 : 4;  // B fragments per wave: (gate, up) x 2, 2, or 4
  f32x16 acc[2][NB];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][nb][r] = 0.f;

  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 31, fk = (lane >> 5) * 8;
  // 32-row MFMA blocks that lie wholly past the segment's last row hold only padding: their
  // waves skip the fragment reads and products (wave-uniform), which leaves them zero
  const int live_mi = (tc.row0 + wm * 64 < tc.row_end) + (tc.row0 + wm * 64 + 32 < tc.row_end);

  load_tile(0);
  store_tile();
  __syncthreads();
  const int nk = KD / BK;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_tile((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      if (live_mi == 0) break;
      u32x4 af[2], bfr[NB];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        if (mi < live_mi) af[mi] = ld16(a_lds + (wm * 64 + mi * 32 + frow) * LDS_STRIDE + kk + fk);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        // stage 0: nb 0,1 -> gate rows, nb 2,3 -> up rows of the same columns; stage 2: nb 2,3 ->
        // the tile's second 128 columns
        const int brow = (STAGE != 1 && nb >= 2 ? BN : 0) + wn * 64 + (nb & 1) * 32 + frow;
        bfr[nb] = ld16(b_lds + brow * LDS_STRIDE + kk + fk);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        if (mi >= live_mi) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mi][nb] = mfma_32x32x16_bf16(af[mi], bfr[nb], acc[mi][nb]);
      }
    }
    __syncthreads();
    if (kt + 1 < nk) {
      store_tile();
      __syncthreads();
    }
  }

  // ---- epilogue.  32x32 MFMA D layout: lane l, item r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
  uint16_t* out = static_cast<uint16_t*>(sh ? g.sh_out : g.out);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = tc.row0 + wm * 64 + mi * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
      if (row >= tc.row_end) continue;
#pragma unroll
      for (int ni = 0; ni < (STAGE == 2 ? 4 : 2); ++ni) {
        const int col = n0 + (ni >= 2 ? BN : 0) + wn * 64 + (ni & 1) * 32 + (lane % 32);
        float v;
        if (STAGE == 0) v = silu(acc[mi][ni][r]) * acc[mi][ni + 2][r];
        else v = acc[mi][ni][r];
        out[(size_t)row * NCOLS + col] = (uint16_t)f32_to_bf16(v);
      }
    }
}

}  // namespace

hipError_t launch_grouped_gemm_bf16(const GroupedGemmArgs& g, hipStream_t s) {
  if (g.N == 0) return hipSuccess;
  if (!g.row_invariant && decode_gemm_fits(g)) return launch_grouped_gemm_decode(g, s);
  if (g.stage == 0) {
    k_grouped_gemm_bf16<0><<<grouped_grid(g, gemm_groups(g, 0, BN), BM), 256, 0, s>>>(g);
  } else if (g.H % (2 * BN) == 0) {
    k_grouped_gemm_bf16<2><<<grouped_grid(g, gemm_groups(g, 1, 2 * BN), BM), 256, 0, s>>>(g);
  } else {
    k_grouped_gemm_bf16<1><<<grouped_grid(g, gemm_groups(g, 1, BN), BM), 256, 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace moe
