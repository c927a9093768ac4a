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
// 64 x 64 (x2 for gate and up).  The operands stream through an LDS ring filled
// by direct global -> LDS loads (A and B rows in 16-byte pieces, XOR-swizzled;
// the weight rows' E8M0 codes and the activation rows' fp32 scales of each step
// in 4-byte pieces), several K steps ahead of the MFMAs, so the loads in flight
// hold no registers.  The gate/up epilogue computes h = silu(g) * u and
// quantises it per row over the tile's 128 columns to e4m3 (the recipe of
// moe_quantize_fp8); the down stage writes bf16.
#include "common.h"
#include "dma.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int E8M0_ONE = 127;  // E8M0 code of 2^0

// Waves per block: gate/up 16 (four per SIMD, one block per CU, 32 x 32 wave tiles x gate and up;
// 4 waves ran 1,467 us, 8 ran 1,255 and 16 ran 1,228 on the DeepSeek-like layer); down 4 (two blocks
// per CU).
constexpr int MX_GU_WAVES = 16, MX_DN_WAVES = 4;

// WIN: the scales travel in windows of 4 K steps (WIN_STEPS) instead of with every step: each weight
// row's 16 E8M0 codes and each activation row's 4 fp32 scales of a window are one contiguous 16-byte
// piece, so a window costs one L2 request per row where per-step loads cost one per row and step.  A
// window's pieces are loaded in WIN_STEPS slices, one with each ring stage of the window before it, into
// one of three window buffers (a buffer is rewritten only after every step of the window it held is
// done).  Needs whole windows: KD / BK a multiple of WIN_STEPS.
constexpr int WIN_STEPS = 4, WIN_BUFS = 3;

template <int STAGE, bool WIN = false>
struct MxShape {
  static constexpr int WAVES = STAGE == 0 ? MX_GU_WAVES : MX_DN_WAVES;
  static constexpr int WN = WAVES == 4 ? 2 : 4;           // waves along the columns
  static constexpr int WM = WAVES / WN;                   // ... along the rows
  static constexpr int MI = BM / WM / 32;                 // 32-row MFMA blocks per wave
  static constexpr int NI = BN / WN / 32;                 // 32-column blocks per wave (x2 gate/up)
  static constexpr int BROWS = STAGE == 0 ? 2 * BN : BN;  // weight rows per tile
  static constexpr int NSTAGE = STAGE == 0 ? 4 : 3;       // gate/up: one block per CU; down: two
  static constexpr int ABYTES = BM * BK;                  // e4m3 rows
  static constexpr int BBYTES = BROWS * BK / 2;           // packed E2M1 rows
  static constexpr int BSBYTES = BROWS * 4;               // the 4 E8M0 codes of each weight row
  static constexpr int ASBYTES = BM * 4;                  // the fp32 scale of each activation row
  static constexpr int SBYTES = ABYTES + BBYTES + (WIN ? 0 : BSBYTES + ASBYTES);
  static constexpr int A_DMA = ABYTES / 1024 / WAVES;     // 16-byte A loads per wave per step
  static constexpr int B_DMA = BBYTES / 1024 / WAVES;     // 16-byte B loads per wave per step
  static constexpr int VM = A_DMA + B_DMA + (WIN ? 1 : 2);  // load instructions per wave per step
  // WIN: a window holds one 16-byte piece per weight row and per activation row; slice j of it (loaded
  // with one ring stage) covers rows SLICE_ROWS j .., PPW rows per wave
  static constexpr int WIN_ROWS = BROWS + BM;
  static constexpr int WIN_BYTES = WIN_ROWS * 16;
  static constexpr int SLICE_ROWS = WIN_ROWS / WIN_STEPS;
  static constexpr int PPW = SLICE_ROWS / WAVES;
  static_assert(!WIN || (SLICE_ROWS * WIN_STEPS == WIN_ROWS && PPW * WAVES == SLICE_ROWS && 4 * PPW <= kWave),
                "window slices");
  static constexpr int LDS = NSTAGE * SBYTES + (WIN ? WIN_BUFS * WIN_BYTES : 0);
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ void dma4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)lds_base, 4, 0, 0);
}

// wait until at most `stages_after` later steps (VM loads each) are still in flight
template <int NSTAGE, int VM>
__device__ __forceinline__ void wait_steps(int stages_after) {
  static_assert(NSTAGE == 3 || NSTAGE == 4, "one case per possible count of later steps");
  if (stages_after == 0) dma_wait<0>();
  else if (NSTAGE == 3 || stages_after == 1) dma_wait<VM>();
  else dma_wait<(NSTAGE == 4 ? 2 * VM : VM)>();
}

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

template <int STAGE, bool WIN>
__global__ __launch_bounds__(MxShape<STAGE>::WAVES * 64, STAGE == 0 ? 1 : 2) void k_grouped_gemm_mxfp4(GroupedGemmArgs g) {
  using S = MxShape<STAGE, WIN>;
  constexpr int NSTAGE = S::NSTAGE, VM = S::VM, BROWS = S::BROWS, MI = S::MI, NI = S::NI;
  constexpr int WR = BM / S::WM, WC = BN / S::WN;  // a wave's tile rows and columns
  extern __shared__ __align__(16) uint8_t smem[];  // S::LDS bytes: the ring
  int* s_prefix = reinterpret_cast<int*>(smem);     // scheduler scratch, dead before the first load
  int* s_wsum = s_prefix + kMaxGroups + 1;

  const Groups G = gemm_groups(g, STAGE, BN);
  const TileCoord tc = schedule_tile(G, BM, s_prefix, s_wsum);
  if (tc.expert < 0) return;  // the same decision in every thread
  const bool sh = tc.expert == G.nr;  // the shared expert's group
  const int KD = STAGE == 0 ? g.H : (sh ? g.Is : g.I);
  const int NCOLS = STAGE == 0 ? (sh ? g.Is : g.I) : g.H;
  const int KB = KD / BK;
  __syncthreads();            // every wave is done with the scheduler scratch before the loads reuse it

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n0 = tc.n_tile * BN;

  const uint8_t *wa, *wb = nullptr;      // packed codes [rows, KD/2]
  const uint8_t *sa_w, *sb_w = nullptr;  // E8M0 codes [rows, KD/32]
  if (STAGE == 0) {
    wa = static_cast<const uint8_t*>(sh ? g.sh_gate : g.w_gate[tc.expert]);
    wb = static_cast<const uint8_t*>(sh ? g.sh_up : g.w_up[tc.expert]);
    sa_w = reinterpret_cast<const uint8_t*>(sh ? g.sh_gate_s : g.s_gate[tc.expert]);
    sb_w = reinterpret_cast<const uint8_t*>(sh ? g.sh_up_s : g.s_up[tc.expert]);
  } else {
    wa = static_cast<const uint8_t*>(sh ? g.sh_down : g.w_down[tc.expert]);
    sa_w = reinterpret_cast<const uint8_t*>(sh ? g.sh_down_s : g.s_down[tc.expert]);
  }
  auto weight_row = [&](int r, const uint8_t* base_a, const uint8_t* base_b, size_t row_bytes) {
    if (STAGE == 0) return r < BN ? base_a + (size_t)(n0 + r) * row_bytes : base_b + (size_t)(n0 + r - BN) * row_bytes;
    return base_a + (size_t)(n0 + r) * row_bytes;
  };
  auto a_row = [&](int trow) {  // the x / h row behind tile row trow
    int p = tc.row0 + trow;
    if (p >= tc.row_end) p = tc.row_end - 1;  // rows past the segment are computed, never stored
    return STAGE == 0 ? (sh ? (long)p : (long)(g.sorted_ids[p] / g.K)) : (long)p;
  };

  // Load sources.  A: instruction i of wave w writes tile rows 8 (4 w + i) .. + 7, lane l row
  // + l / 8 at 16-byte slot l % 8, which holds memory chunk (l % 8) ^ ((row / 2) % 8).  B:
  // instruction i writes weight rows 16 (B_DMA w + i) .. + 15, lane l row + l / 4 at slot l % 4 =
  // chunk (l % 4) ^ ((row / 4) % 4).  A fragment read serves 16 lanes (16 consecutive rows, one
  // chunk) per LDS cycle; these swizzles put them in 16 different 16-byte bank groups.  Scales: 4-byte pieces, the weight rows' E8M0 words (gate/up: 64 rows per
  // wave; down: 32) and the activation rows' fp32 scales (32 rows per wave), row r at 4 r.
  const uint8_t* a_src = static_cast<const uint8_t*>(sh ? g.sh_a : g.a);
  const uint8_t* a_ptr[S::A_DMA];
#pragma unroll
  for (int i = 0; i < S::A_DMA; ++i) {
    const int trow = (S::A_DMA * wave + i) * 8 + lane / 8;
    a_ptr[i] = a_src + (size_t)a_row(trow) * KD + (((lane % 8) ^ ((trow >> 1) & 7)) << 4);
  }
  const uint8_t* b_ptr[S::B_DMA];
#pragma unroll
  for (int i = 0; i < S::B_DMA; ++i) {
    const int wr = (S::B_DMA * wave + i) * 16 + lane / 4;
    b_ptr[i] = weight_row(wr, wa, wb, (size_t)KD / 2) + (((lane % 4) ^ ((wr >> 2) & 3)) << 4);
  }
  const int bs_rows = BROWS / S::WAVES;  // E8M0 rows per wave
  const bool bs_lane = lane < bs_rows;
  const uint8_t* bs_ptr = weight_row(bs_lane ? wave * bs_rows + lane : 0, sa_w, sb_w, (size_t)KD / 32);
  const int as_rows = BM / S::WAVES;  // activation-scale rows per wave
  const bool as_lane = lane < as_rows;
  const float* as_ptr = (sh ? g.sh_a_scales : g.a_scales) + (size_t)a_row(as_lane ? wave * as_rows + lane : 0) * KB;

  // WIN: with slice j, lanes 4 i .. 4 i + 3 (i < PPW) of wave w load the window piece of row
  // rho = SLICE_ROWS j + PPW w + i (weight rows first, then activation rows) as four 4-byte words, which
  // the address unit joins into one request; win_src[j] is the lane's word of window 0
  uint8_t* const win_lds = smem + NSTAGE * S::SBYTES;
  const uint8_t* win_src[WIN ? WIN_STEPS : 1];
  if constexpr (WIN) {
#pragma unroll
    for (int j = 0; j < WIN_STEPS; ++j) {
      const int rho = min(S::SLICE_ROWS * j + S::PPW * wave + lane / 4, S::WIN_ROWS - 1);
      win_src[j] = (rho < BROWS ? weight_row(rho, sa_w, sb_w, (size_t)KD / 32)
                                : reinterpret_cast<const uint8_t*>((sh ? g.sh_a_scales : g.a_scales) +
                                                                   (size_t)a_row(rho - BROWS) * KB)) +
                   (lane % 4) * 4;
    }
  }
  auto issue_slice = [&](int v, int j) {  // slice j of window v (v past the last: the last again, unused)
    const int vs = min(v, KB / WIN_STEPS - 1);
    if (lane < 4 * S::PPW)
      dma4(win_src[j] + (size_t)vs * 16, win_lds + (v % WIN_BUFS) * S::WIN_BYTES + (S::SLICE_ROWS * j + S::PPW * wave) * 16);
  };

  auto issue = [&](int buf, int kb) {
    uint8_t* sa = smem + buf * S::SBYTES;
    uint8_t* sb = sa + S::ABYTES;
    uint8_t* sbs = sb + S::BBYTES;
    uint8_t* sas = sbs + S::BSBYTES;
#pragma unroll
    for (int i = 0; i < S::A_DMA; ++i) dma16(a_ptr[i] + (size_t)kb * BK, sa + (S::A_DMA * wave + i) * 1024);
#pragma unroll
    for (int i = 0; i < S::B_DMA; ++i) dma16(b_ptr[i] + (size_t)kb * (BK / 2), sb + (S::B_DMA * wave + i) * 1024);
    if constexpr (WIN) {
      // slice kb % 4 of window kb / 4 + 1: that buffer last held window kb / 4 - 2, whose last step,
      // 4 (kb / 4) - 5, every wave has finished by the barrier of step kb - 3 that precedes this issue
      issue_slice(kb / WIN_STEPS + 1, kb % WIN_STEPS);
    } else {
      if (bs_lane) dma4(bs_ptr + (size_t)kb * 4, sbs + wave * bs_rows * 4);
      if (as_lane) dma4(as_ptr + kb, sas + wave * as_rows * 4);
    }
  };

  constexpr int NB = STAGE == 0 ? 2 * NI : NI;
  f32x16 acc[MI][NB];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][nb][r] = 0.f;

  const int wm = wave / S::WN, wn = wave % S::WN;
  const int frow = lane & 31, half = lane >> 5;  // the lane's row and half of a 64-wide MFMA step
  auto item_row = [&](int r) { return 8 * (r / 4) + 4 * half + (r % 4); };
  // 32-row MFMA blocks that lie wholly past the segment's last row hold only padding: their
  // waves skip the fragment reads and products (wave-uniform), which leaves them zero
  int live_mi = 0;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) live_mi += tc.row0 + wm * WR + mi * 32 < tc.row_end;

  if constexpr (WIN) {
#pragma unroll
    for (int j = 0; j < WIN_STEPS; ++j) issue_slice(0, j);  // window 0, older than every ring stage
  }
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < KB) issue(s, s);

  for (int kb = 0; kb < KB; ++kb) {
    const int later = KB - 1 - kb;  // steps issued after step kb (capped by the ring depth)
    wait_steps<NSTAGE, VM>(later < NSTAGE - 2 ? later : NSTAGE - 2);
    __builtin_amdgcn_s_barrier();  // step kb has landed in every wave; every wave is done with kb - 1
    __builtin_amdgcn_sched_barrier(0);
    if (kb + NSTAGE - 1 < KB) issue((kb + NSTAGE - 1) % NSTAGE, kb + NSTAGE - 1);
    if (live_mi == 0) continue;
    const uint8_t* sa = smem + (kb % NSTAGE) * S::SBYTES;
    const uint8_t* sb = sa + S::ABYTES;
    // this step's 4 E8M0 codes of weight row r and fp32 scale of activation row r
    const uint8_t* win = win_lds + ((kb / WIN_STEPS) % WIN_BUFS) * S::WIN_BYTES + (kb % WIN_STEPS) * 4;
    auto bcodes = [&](int r) {
      return WIN ? *reinterpret_cast<const uint32_t*>(win + r * 16)
                 : reinterpret_cast<const uint32_t*>(sb + S::BBYTES)[r];
    };
    auto ascale = [&](int r) {
      return WIN ? *reinterpret_cast<const float*>(win + (BROWS + r) * 16)
                 : reinterpret_cast<const float*>(sb + S::BBYTES + S::BSBYTES)[r];
    };
    f32x16 blk[MI][NB];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) blk[mi][nb][r] = 0.f;
    // fragment reads and MFMAs at raised wave priority: a wave whose operands are ready issues ahead of
    // the waves in their scale promotions (back to normal priority before its own promotions)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 64) {
      i32x8 af[MI], bfr[NB];
      int bsc[NB];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        if (mi >= live_mi) continue;
        const int ar = wm * WR + mi * 32 + frow;
        const uint8_t* rowp = sa + ar * BK;
        const int c1 = kk / 16 + half, c2 = kk / 16 + 2 + half;  // memory K 16 h and 32 + 16 h
        const u32x4 lo = *reinterpret_cast<const u32x4*>(rowp + ((c1 ^ ((ar >> 1) & 7)) << 4));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(rowp + ((c2 ^ ((ar >> 1) & 7)) << 4));
        af[mi] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        // stage 0: nb < NI -> gate rows, nb >= NI -> up rows of the same columns
        const int wr = (STAGE == 0 && nb >= NI ? BN : 0) + wn * WC + (nb % NI) * 32 + frow;
        const int c = kk / 32 + half;  // memory block of the lane's 32 codes (16 bytes)
        const u32x4 v = *reinterpret_cast<const u32x4*>(sb + wr * (BK / 2) + ((c ^ ((wr >> 2) & 3)) << 4));
        bfr[nb] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        bsc[nb] = (int)((bcodes(wr) >> (8 * c)) & 0xFFu);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        if (mi >= live_mi) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) blk[mi][nb] = mfma_e4m3_x_e2m1(af[mi], bfr[nb], bsc[nb], blk[mi][nb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // promote this K step: acc += blk * (activation row scale); the weight scales are inside blk
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (mi >= live_mi) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float rs = ascale(wm * WR + mi * 32 + item_row(r));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mi][nb][r] += blk[mi][nb][r] * rs;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  if (STAGE == 1) {
    uint16_t* out = static_cast<uint16_t*>(sh ? g.sh_out : g.out);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tc.row0 + wm * WR + mi * 32 + item_row(r);
        if (row >= tc.row_end) continue;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int col = n0 + wn * WC + ni * 32 + (lane % 32);
          out[(size_t)row * NCOLS + col] = (uint16_t)f32_to_bf16(acc[mi][ni][r]);
        }
      }
    return;
  }

  // ---- gate/up epilogue: h = silu(g) * u, quantised per row over this tile's 128 columns.  The h
  // values go through LDS (the ring is free) so that each row is finished by the threads that hold
  // it: an amax over a few lanes, and the codes leave as 4-byte stores.
  __syncthreads();  // every wave is past its last ring read
  constexpr int HSTRIDE = BN + 4;  // floats per LDS row (4 of padding: rows 4 apart fall on other banks)
  float* h_lds = reinterpret_cast<float*>(smem);  // [BM][HSTRIDE]
  static_assert(BM * HSTRIDE * 4 <= S::LDS, "h fits in the ring");
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        h_lds[(wm * WR + mi * 32 + item_row(r)) * HSTRIDE + wn * WC + ni * 32 + (lane % 32)] =
            silu(acc[mi][ni][r]) * acc[mi][ni + NI][r];
  __syncthreads();
  uint8_t* out = static_cast<uint8_t*>(sh ? g.sh_out : g.out);
  float* out_scales = sh ? g.sh_out_scales : g.out_scales;
  const int groups = NCOLS / 128;
  constexpr int TPR = S::WAVES * 64 / BM;  // threads per row
  constexpr int VPT = BN / TPR;            // values per thread
  static_assert(TPR * VPT == BN && VPT % 4 == 0 && (TPR & (TPR - 1)) == 0 && TPR <= kWave, "row split");
  const int trow = threadIdx.x / TPR, seg = threadIdx.x % TPR;
  // thread seg of a row holds the float4 groups at columns 4 seg + 4 TPR i: the row's threads read one
  // contiguous span per instruction
  float v[VPT];
#pragma unroll
  for (int i = 0; i < VPT / 4; ++i) {
    const f32x4 q = *reinterpret_cast<const f32x4*>(h_lds + trow * HSTRIDE + 4 * seg + 4 * TPR * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[4 * i + j] = q[j];
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
  const int row = tc.row0 + trow;
  if (row < tc.row_end) {
    const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
#pragma unroll
    for (int i = 0; i < VPT / 4; ++i) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) word |= f32_to_e4m3(v[4 * i + j] * inv) << (8 * j);
      *reinterpret_cast<uint32_t*>(out + (size_t)row * NCOLS + n0 + 4 * seg + 4 * TPR * i) = word;
    }
    if (seg == 0) out_scales[(size_t)row * groups + tc.n_tile] = amax > 0.f ? amax / 448.0f : 1.0f;
  }
}

// ---- the down stage with persistent blocks, two per CU
//
// The same tiles, ring (three stages, the E8M0 codes and activation scales of each step riding in it),
// MFMAs and promotions as k_grouped_gemm_mxfp4<1, false>, so the same bits; but block b of XCD x =
// b % 8 walks the tiles b / 8, b / 8 + S, ... (S blocks per XCD) of that XCD's contiguous range of
// logical tiles, and the ring does not drain between them: the last two K steps of a tile issue the next
// tile's first two stages.  The tile prefix is built once per block (it stays in LDS after the ring).
// A down tile streams 16 K steps in ~13 us, so the one-tile-per-block kernel's scheduler, first-stage
// latency and epilogue are a large share of its time.
using MxDn = MxShape<1, false>;
constexpr int MXP_PREFIX_OFF = MxDn::NSTAGE * MxDn::SBYTES;
constexpr int MXP_LDS = MXP_PREFIX_OFF + (kMaxGroups + 1 + kMaxSchedWaves) * 4;
static_assert(2 * MXP_LDS <= 160 * 1024, "two blocks per CU");

struct MxDownTile {
  int expert, n_tile, row0, row_end, KB, live_mi, sh;
  const uint8_t* a_ptr[MxDn::A_DMA];
  const uint8_t* b_ptr[MxDn::B_DMA];
  const uint8_t* bs_ptr;
  const float* as_ptr;
};

__global__ __launch_bounds__(MX_DN_WAVES * 64, 2) void k_grouped_gemm_mxfp4_down_persistent(GroupedGemmArgs g) {
  using S = MxDn;
  constexpr int NSTAGE = S::NSTAGE, VM = S::VM, MI = S::MI, NI = S::NI;
  constexpr int WR = BM / S::WM, WC = BN / S::WN;
  extern __shared__ __align__(16) uint8_t smem[];
  int* s_prefix = reinterpret_cast<int*>(smem + MXP_PREFIX_OFF);
  int* s_wsum = s_prefix + kMaxGroups + 1;

  __shared__ int s_next;

  const Groups G = gemm_groups(g, 1, BN);
  const int T = tile_prefix(G, BM, s_prefix, s_wsum);
  const int SB = (int)gridDim.x / 8, x = blockIdx.x % 8;  // blocks per XCD; this block's XCD
  const int chunk = (T + 7) / 8;
  const int t0 = x * chunk, t_end = min((x + 1) * chunk, T);
  int L = t0 + (int)blockIdx.x / 8;
  if (L >= t_end) return;  // the same decision in every thread
  // with the launch's tile counters (g.queue): the XCD's nT tiles, the first nb of them taken by its
  // blocks' first tiles; the i-th add on the XCD's counter hands out tile t0 + nb + i, and the add that
  // returns nT - 1 is the XCD's last (each tile a block takes is followed by one add), which puts the
  // counter back to zero.  A block adds at a tile's first K step and reads the answer half a tile later.
  const int nT = t_end - t0, nb = min(SB, nT);
  int32_t* const qw = g.queue != nullptr ? g.queue + x : nullptr;

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = wave / S::WN, wn = wave % S::WN;
  const int frow = lane & 31, half = lane >> 5;
  auto item_row = [&](int r) { return 8 * (r / 4) + 4 * half + (r % 4); };
  const int bs_rows = S::BROWS / S::WAVES;  // E8M0 rows per wave
  const bool bs_lane = lane < bs_rows;
  const int as_rows = BM / S::WAVES;        // activation-scale rows per wave
  const bool as_lane = lane < as_rows;

  // tile Lt: its place and this lane's load sources (as the one-tile kernel computes them)
  auto prepare = [&](int Lt, MxDownTile& t) {
    const TileCoord tc = tile_at_uniform(G, BM, s_prefix, T, Lt);
    t.expert = __builtin_amdgcn_readfirstlane(tc.expert);
    t.n_tile = __builtin_amdgcn_readfirstlane(tc.n_tile);
    t.row0 = __builtin_amdgcn_readfirstlane(tc.row0);
    t.row_end = __builtin_amdgcn_readfirstlane(tc.row_end);
    t.sh = t.expert == G.nr;
    const int KD = t.sh ? g.Is : g.I;
    t.KB = KD / BK;
    t.live_mi = 0;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) t.live_mi += t.row0 + wm * WR + mi * 32 < t.row_end;
    auto a_row = [&](int trow) -> long {
      int p = t.row0 + trow;
      if (p >= t.row_end) p = t.row_end - 1;  // rows past the segment are computed, never stored
      return p;
    };
    const uint8_t* a_src = static_cast<const uint8_t*>(t.sh ? g.sh_a : g.a);
#pragma unroll
    for (int i = 0; i < S::A_DMA; ++i) {
      const int trow = (S::A_DMA * wave + i) * 8 + lane / 8;
      t.a_ptr[i] = a_src + (size_t)a_row(trow) * KD + (((lane % 8) ^ ((trow >> 1) & 7)) << 4);
    }
    const uint8_t* wd = static_cast<const uint8_t*>(t.sh ? g.sh_down : table_entry_uniform(g.w_down, t.expert));
    const uint8_t* sd =
        reinterpret_cast<const uint8_t*>(t.sh ? g.sh_down_s : table_entry_uniform(g.s_down, t.expert));
    const int n0 = t.n_tile * BN;
#pragma unroll
    for (int i = 0; i < S::B_DMA; ++i) {
      const int wr = (S::B_DMA * wave + i) * 16 + lane / 4;
      t.b_ptr[i] = wd + (size_t)(n0 + wr) * (KD / 2) + (((lane % 4) ^ ((wr >> 2) & 3)) << 4);
    }
    t.bs_ptr = sd + (size_t)(n0 + (bs_lane ? wave * bs_rows + lane : 0)) * (KD / 32);
    t.as_ptr = (t.sh ? g.sh_a_scales : g.a_scales) + (size_t)a_row(as_lane ? wave * as_rows + lane : 0) * t.KB;
  };
  auto issue = [&](const MxDownTile& t, int slot, int kb) {
    uint8_t* sa = smem + slot * S::SBYTES;
    uint8_t* sb = sa + S::ABYTES;
    uint8_t* sbs = sb + S::BBYTES;
    uint8_t* sas = sbs + S::BSBYTES;
#pragma unroll
    for (int i = 0; i < S::A_DMA; ++i) dma16(t.a_ptr[i] + (size_t)kb * BK, sa + (S::A_DMA * wave + i) * 1024);
#pragma unroll
    for (int i = 0; i < S::B_DMA; ++i) dma16(t.b_ptr[i] + (size_t)kb * (BK / 2), sb + (S::B_DMA * wave + i) * 1024);
    if (bs_lane) dma4(t.bs_ptr + (size_t)kb * 4, sbs + wave * bs_rows * 4);
    if (as_lane) dma4(t.as_ptr + kb, sas + wave * as_rows * 4);
  };

  MxDownTile cur, nxt;
  prepare(L, cur);
  int gs = 0;  // ring stage of the current tile's K step 0
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < cur.KB) issue(cur, s, s);

  for (;;) {
    int Lnext = -1;
    bool has_next = false;
    bool cross = false;  // the next tile's first stages come from this tile's last two steps
    // counters: the next tile is known from the barrier of step pub (at most KB - 2, so that its stages
    // can still be issued from this tile's last two steps), or, for a tile of under 4 steps, after it
    const int pub = cur.KB >= 4 ? cur.KB / 2 : -1;
    if (qw == nullptr) {
      Lnext = L + SB;
      has_next = Lnext < t_end;
      if (has_next) {
        prepare(Lnext, nxt);
        cross = cur.KB >= NSTAGE - 1 && nxt.KB >= NSTAGE - 1;
      }
    }
    int grab = 0;
    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int nb = 0; nb < NI; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][nb][r] = 0.f;

    for (int kb = 0; kb < cur.KB; ++kb) {
      const int later = cross ? 1 : (kb + 1 < cur.KB ? 1 : 0);  // a stage was issued after step kb
      wait_steps<NSTAGE, VM>(later);
      __builtin_amdgcn_s_barrier();  // step kb has landed in every wave; every wave is done with kb - 1
      __builtin_amdgcn_sched_barrier(0);
      if (qw != nullptr && kb == pub) {
        Lnext = s_next;
        has_next = Lnext >= 0;
        if (has_next) {
          prepare(Lnext, nxt);
          cross = nxt.KB >= NSTAGE - 1;
        }
      }
      if (kb + NSTAGE - 1 < cur.KB) issue(cur, (gs + kb + NSTAGE - 1) % NSTAGE, kb + NSTAGE - 1);
      else if (cross) issue(nxt, (gs + kb + NSTAGE - 1) % NSTAGE, kb + NSTAGE - 1 - cur.KB);
      if (qw != nullptr && threadIdx.x == 0) {
        if (kb == 0) grab = __hip_atomic_fetch_add(qw, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (kb == (pub >= 0 ? pub - 1 : cur.KB - 1)) {  // read by every thread after the next barrier
          s_next = nb + grab < nT ? t0 + nb + grab : -1;
          if (grab == nT - 1) __hip_atomic_store(qw, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (cur.live_mi == 0) continue;
      const uint8_t* sa = smem + ((gs + kb) % NSTAGE) * S::SBYTES;
      const uint8_t* sb = sa + S::ABYTES;
      const uint32_t* bcodes = reinterpret_cast<const uint32_t*>(sb + S::BBYTES);
      const float* ascale = reinterpret_cast<const float*>(sb + S::BBYTES + S::BSBYTES);
      f32x16 blk[MI][NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nb = 0; nb < NI; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) blk[mi][nb][r] = 0.f;
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < BK; kk += 64) {
        i32x8 af[MI], bfr[NI];
        int bsc[NI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          if (mi >= cur.live_mi) continue;
          const int ar = wm * WR + mi * 32 + frow;
          const uint8_t* rowp = sa + ar * BK;
          const int c1 = kk / 16 + half, c2 = kk / 16 + 2 + half;
          const u32x4 lo = *reinterpret_cast<const u32x4*>(rowp + ((c1 ^ ((ar >> 1) & 7)) << 4));
          const u32x4 hi = *reinterpret_cast<const u32x4*>(rowp + ((c2 ^ ((ar >> 1) & 7)) << 4));
          af[mi] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
#pragma unroll
        for (int nb = 0; nb < NI; ++nb) {
          const int wr = wn * WC + nb * 32 + frow;
          const int c = kk / 32 + half;
          const u32x4 v = *reinterpret_cast<const u32x4*>(sb + wr * (BK / 2) + ((c ^ ((wr >> 2) & 3)) << 4));
          bfr[nb] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
          bsc[nb] = (int)((bcodes[wr] >> (8 * c)) & 0xFFu);
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          if (mi >= cur.live_mi) continue;
#pragma unroll
          for (int nb = 0; nb < NI; ++nb) blk[mi][nb] = mfma_e4m3_x_e2m1(af[mi], bfr[nb], bsc[nb], blk[mi][nb]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        if (mi >= cur.live_mi) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float rs = ascale[wm * WR + mi * 32 + item_row(r)];
#pragma unroll
          for (int nb = 0; nb < NI; ++nb) acc[mi][nb][r] += blk[mi][nb][r] * rs;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    {
      uint16_t* out = static_cast<uint16_t*>(cur.sh ? g.sh_out : g.out);
      const int n0 = cur.n_tile * BN;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = cur.row0 + wm * WR + mi * 32 + item_row(r);
          if (row >= cur.row_end) continue;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            out[(size_t)row * g.H + n0 + wn * WC + ni * 32 + (lane % 32)] = (uint16_t)f32_to_bf16(acc[mi][ni][r]);
        }
    }

    if (qw != nullptr && pub < 0) {  // a short tile: its next is read here
      __syncthreads();
      Lnext = s_next;
      has_next = Lnext >= 0;
      if (has_next) prepare(Lnext, nxt);
    }
    if (!has_next) break;
    gs += cur.KB;
    L = Lnext;
    const bool was_cross = cross;
    cur = nxt;
    if (!was_cross) {
      // a short tile on either side: the ring drained (the last step waited for everything); every wave
      // must be past its last ring read before the next tile's first stages overwrite the ring
      __syncthreads();
#pragma unroll
      for (int s = 0; s < NSTAGE - 1; ++s)
        if (s < cur.KB) issue(cur, (gs + s) % NSTAGE, s);
    }
  }
}

}  // namespace

template <int STAGE, bool WIN>
static hipError_t launch_mx(const GroupedGemmArgs& g, hipStream_t s) {
  using S = MxShape<STAGE, WIN>;
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_grouped_gemm_mxfp4<STAGE, WIN>), S::LDS);
  if (e != hipSuccess) return e;
  k_grouped_gemm_mxfp4<STAGE, WIN><<<grouped_grid(g, gemm_groups(g, STAGE, BN), BM), S::WAVES * 64, S::LDS, s>>>(g);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_mxfp4(const GroupedGemmArgs& g, hipStream_t s) {
  if (g.N == 0) return hipSuccess;
  if (g.stage == 0) {
    // scale windows when every group's K steps come in whole windows (K = H for all of them)
    if ((g.H / BK) % WIN_STEPS == 0) return launch_mx<0, true>(g, s);
    return launch_mx<0, false>(g, s);
  }
  // down: persistent blocks, two per CU, a multiple of 8 (the XCDs) and no more than the tiles can use
  const int cus = device_cus();
  if (cus >= 8) {
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_grouped_gemm_mxfp4_down_persistent), MXP_LDS);
    if (e != hipSuccess) return e;
    unsigned grid = (unsigned)(2 * cus / 8 * 8);
    const unsigned tiles = grouped_grid(g, gemm_groups(g, 1, BN), BM);  // a multiple of 8
    if (tiles < grid) grid = tiles;
    k_grouped_gemm_mxfp4_down_persistent<<<grid, MX_DN_WAVES * 64, MXP_LDS, s>>>(g);
    return hipGetLastError();
  }
  return launch_mx<1, false>(g, s);
}

}  // namespace moe
