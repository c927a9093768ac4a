// Grouped expert GEMMs on OCP e4m3 weights with fp32 128x128 block scales, for
// gfx950 (v_mfma_f32_32x32x64_f8f6f4, e4m3 x e4m3 -> fp32).
//
// Same data flow as the bf16 kernels (forward_prefill.rs page,
// run_routed_grouped_gemm; the FP8 expert tables of the forward.rs page carry
// one weight pointer and one scale pointer per expert).  The activation rows
// carry one fp32 scale per 128 columns and the weights one per 128x128 block,
// neither of which is the power-of-two block scale the scaled MFMA consumes, so
// every K step is exactly one 128-column scale block: its MFMA sums start from
// zero, and the block result is promoted into the fp32 accumulator with the
// product (row scale x weight-block scale) on the vector ALU.
//
// Block tile BM = 128 rows x BN = 128 output columns, K step 128 bytes, 4 waves
// in 2 x 2, each wave 64 x 64 (x2 for gate and up).  The gate/up epilogue
// computes h = silu(g) * u and quantises it per row over the tile's 128 columns
// (one e4m3 scale group, the same recipe as moe_quantize_fp8), so h leaves the
// kernel as e4m3 codes + one fp32 scale per 128 columns.
#include "common.h"
#include "dma.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDS_STRIDE = BK + 16;  // bytes per LDS row

template <int STAGE>
struct Fp8Tile {
  static constexpr int BROWS = STAGE == 0 ? 2 * BN : BN;
  static constexpr int A_LOADS = BM * (BK / 16) / 256;  // 16-byte chunks per thread
  static constexpr int B_LOADS = BROWS * (BK / 16) / 256;
  static constexpr int LDS_BYTES = (BM + BROWS) * LDS_STRIDE;
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <int STAGE>
__global__ __launch_bounds__(256, STAGE == 0 ? 1 : 2) void k_grouped_gemm_fp8(GroupedGemmArgs g) {
  using T = Fp8Tile<STAGE>;
  __shared__ __align__(16) uint8_t lds[T::LDS_BYTES];
  __shared__ float s_asc[BM];   // row scales of the current K block
  __shared__ float s_amax[2][BM];  // gate/up epilogue: per-row amax of each column half
  uint8_t* a_lds = lds;
  uint8_t* b_lds = lds + BM * LDS_STRIDE;
  __shared__ int s_prefix[kMaxGroups + 1];
  __shared__ int s_wsum[4];

  const Groups G = gemm_groups(g, STAGE, BN);
  const TileCoord tc = schedule_tile(G, BM, s_prefix, s_wsum, 32);
  if (tc.expert < 0) return;
  const bool sh = tc.expert == G.nr;  // the shared expert's group
  const int KD = STAGE == 0 ? g.H : (sh ? g.Is : g.I);
  const int NCOLS = STAGE == 0 ? (sh ? g.Is : g.I) : g.H;
  const int KB = KD / 128;  // scale blocks along K

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int n0 = tc.n_tile * BN;

  const uint8_t *wa, *wb = nullptr;
  const float *sa_w, *sb_w = nullptr;  // weight block scales
  if (STAGE == 0) {
    wa = static_cast<const uint8_t*>(sh ? g.sh_gate : g.w_gate[tc.expert]);
    wb = static_cast<const uint8_t*>(sh ? g.sh_up : g.w_up[tc.expert]);
    sa_w = sh ? g.sh_gate_s : g.s_gate[tc.expert];
    sb_w = sh ? g.sh_up_s : g.s_up[tc.expert];
  } else {
    wa = static_cast<const uint8_t*>(sh ? g.sh_down : g.w_down[tc.expert]);
    sa_w = sh ? g.sh_down_s : g.s_down[tc.expert];
  }
  // weight scales of this tile's 128 output columns: row block n0/128 of the [NCOLS/128, KB] scale grid
  const float* swa = sa_w + (size_t)(n0 / 128) * KB;
  const float* swb = STAGE == 0 ? sb_w + (size_t)(n0 / 128) * KB : nullptr;

  const uint8_t* a_src = static_cast<const uint8_t*>(sh ? g.sh_a : g.a);
  const float* a_scales = sh ? g.sh_a_scales : g.a_scales;
  const int lrow = tid >> 3;        // 0..31
  const int lcol = (tid & 7) * 16;  // byte column of this thread's 16-byte chunk
  const uint8_t* a_ptr[T::A_LOADS];
#pragma unroll
  for (int i = 0; i < T::A_LOADS; ++i) {
    int p = tc.row0 + lrow + 32 * i;
    if (p >= tc.row_end) p = tc.row_end - 1;
    long arow = STAGE == 0 ? (sh ? p : g.sorted_ids[p] / g.K) : p;
    a_ptr[i] = a_src + (size_t)arow * KD + lcol;
  }
  // the row-scale row of the A row this thread stages (threads 0..127, one row each)
  const float* asc_ptr = nullptr;
  if (tid < BM) {
    int p = tc.row0 + tid;
    if (p >= tc.row_end) p = tc.row_end - 1;
    long arow = STAGE == 0 ? (sh ? p : g.sorted_ids[p] / g.K) : p;
    asc_ptr = a_scales + (size_t)arow * KB;
  }
  const uint8_t* b_ptr[T::B_LOADS];
#pragma unroll
  for (int i = 0; i < T::B_LOADS; ++i) {
    const int r = lrow + 32 * i;
    if (STAGE == 0) b_ptr[i] = (r < BN ? wa + (size_t)(n0 + r) * KD : wb + (size_t)(n0 + r - BN) * KD) + lcol;
    else b_ptr[i] = wa + (size_t)(n0 + r) * KD + lcol;
  }

  u32x4 ra[T::A_LOADS], rb[T::B_LOADS];
  float rsc = 0.f;
  auto load_tile = [&](int kb) {
    const int k0 = kb * BK;
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) ra[i] = ldg16(a_ptr[i] + k0);
#pragma unroll
    for (int i = 0; i < T::B_LOADS; ++i) rb[i] = ldg16(b_ptr[i] + k0);
    if (tid < BM) rsc = ldg_f32(asc_ptr + kb);
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) st16(a_lds + (lrow + 32 * i) * LDS_STRIDE + lcol, ra[i]);
#pragma unroll
    for (int i = 0; i < T::B_LOADS; ++i) st16(b_lds + (lrow + 32 * i) * LDS_STRIDE + lcol, rb[i]);
    if (tid < BM) s_asc[tid] = rsc;
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
  const int frow = lane & 31, fk = (lane >> 5) * 32;
  // rows of this lane's accumulator items (32x32 D layout), relative to the wave's 32-row sub-tile
  auto item_row = [&](int r) { return 8 * (r / 4) + 4 * (lane / 32) + (r % 4); };

  load_tile(0);
  store_tile();
  __syncthreads();
  for (int kb = 0; kb < KB; ++kb) {
    const float wsa = ldg_f32(swa + kb);
    const float wsb = STAGE == 0 ? ldg_f32(swb + kb) : 0.f;
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
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const uint8_t* p = a_lds + (wm * 64 + mi * 32 + frow) * LDS_STRIDE + kk + fk;
        const u32x4 lo = ld16(p), hi = ld16(p + 16);
        af[mi] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int brow = (STAGE == 0 && nb >= 2 ? BN : 0) + wn * 64 + (nb & 1) * 32 + frow;
        const uint8_t* p = b_lds + brow * LDS_STRIDE + kk + fk;
        const u32x4 lo = ld16(p), hi = ld16(p + 16);
        bfr[nb] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) blk[mi][nb] = mfma_32x32x64_fp8(af[mi], bfr[nb], blk[mi][nb]);
    }
    // promote this scale block: acc += blk * (row scale * weight-block scale)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float rs = s_asc[wm * 64 + mi * 32 + item_row(r)];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float ws = (STAGE == 0 && nb >= 2) ? wsb : wsa;
          acc[mi][nb][r] += blk[mi][nb][r] * (rs * ws);
        }
      }
    __syncthreads();
    if (kb + 1 < KB) {
      store_tile();
      __syncthreads();
    }
  }

  if (STAGE == 1) {
    uint16_t* out = static_cast<uint16_t*>(sh ? g.sh_out : g.out);
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
      // max over the 32 lanes that hold this row (same lane / 32)
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
      if ((lane & 31) == 0) s_amax[wn][wm * 64 + mi * 32 + item_row(r)] = m;
    }
  __syncthreads();
  uint8_t* out = static_cast<uint8_t*>(sh ? g.sh_out : g.out);
  float* out_scales = sh ? g.sh_out_scales : g.out_scales;
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
        if (wn == 0 && (lane & 31) == 0)
          out_scales[(size_t)row * groups + tc.n_tile] = amax > 0.f ? amax / 448.0f : 1.0f;
      }
    }
}

// ---- streaming kernel for groups of up to a few hundred rows (the routed experts)
//
// There the GEMM is bound by streaming the weights from HBM, and the MFMAs and
// the per-scale-block promotions must hide under that stream.  A tile spans a
// whole group of up to 128 rows (each weight slab enters LDS once) and 256
// weight rows (gate/up: 128 columns of gate and the same 128 of up, so the
// tile's 128 h columns are one quantisation group; down: 256 output columns, two
// weight-scale blocks).  K step = 128 bytes = one scale block.  The operands go
// through a 3-stage LDS ring filled by direct global -> LDS loads, two steps
// ahead of the MFMAs; the activation rows' scales of each step ride in the ring
// (one 4-byte load per lane and row), the tile's weight-block scales are read
// into LDS once.  Several waves per SIMD, so one wave's promotions overlap
// another's MFMAs: gate/up 16 waves in 4 x 4, each 32 rows x 2 blocks of 32
// weight rows (one gate block and the matching up block); down 8 waves in 2 x 4,
// each 64 rows x 64 columns.  A wave's block sums and accumulators stay in its
// VGPRs, so a promotion is one FMA per value.  Chunk c of LDS row r sits at
// 16-byte slot c ^ ((r / 2) % 8).
constexpr int SBM = 128, SBNB = 256, SROWB = 128, SNSTAGE = 3;
constexpr int SABYTES = SBM * SROWB, SBBYTES = SBNB * SROWB;
constexpr int SSTAGE = SABYTES + SBBYTES + SBM * 4;  // 48.5 KB
// Waves per block: gate/up 16 (four per SIMD, 32 x 64 wave tiles: 1,430 -> 1,358 us on the
// DeepSeek-like layer), down 8 (two per SIMD, 64 x 64; 16 waves ran it 660 -> 684 us).
template <int STAGE>
struct StreamWaves {
  static constexpr int WAVES = STAGE == 0 ? 16 : 8;
  static constexpr int WM = WAVES / 4;     // waves along the rows (4 along the weight rows)
  static constexpr int WR = SBM / WM;      // tile rows per wave
  static constexpr int MI = WR / 32;       // 32-row MFMA blocks per wave
  static constexpr int AR = SBM / WAVES;   // A rows each wave loads per stage
  static constexpr int AI = AR / 8;        // ... in 8-row load instructions
  static constexpr int BR = SBNB / WAVES;  // B rows each wave loads per stage
  static constexpr int BI = BR / 8;
  static constexpr int VM = AI + BI + 1;   // load instructions per wave per stage
};
constexpr int SMAXKB = 64;                           // weight-scale blocks along K held in LDS (K <= 8192)
constexpr int SLDS = SNSTAGE * SSTAGE + 2 * SMAXKB * 4;  // 146 KB: one block per CU

template <int STAGE>
__global__ __launch_bounds__(StreamWaves<STAGE>::WAVES * 64, 1) void k_grouped_gemm_fp8_stream(GroupedGemmArgs g) {
  using W = StreamWaves<STAGE>;
  constexpr int SWR = W::WR, SMI = W::MI, SAR = W::AR, SAI = W::AI, SBR = W::BR, SBI = W::BI, SVM = W::VM;
  extern __shared__ __align__(16) uint8_t smem[];
  int* s_prefix = reinterpret_cast<int*>(smem);  // scheduler scratch, dead before the first load
  int* s_wsum = s_prefix + kMaxGroups + 1;
  float* s_ws = reinterpret_cast<float*>(smem + SNSTAGE * SSTAGE);  // [2][SMAXKB] weight-block scales

  const int COLS = STAGE == 0 ? SBNB / 2 : SBNB;  // output columns per tile
  const Groups G = gemm_groups(g, STAGE, COLS);
  const TileCoord tc = schedule_tile(G, SBM, s_prefix, s_wsum, 32);
  if (tc.expert < 0) return;  // the same decision in every thread
  const bool sh = tc.expert == G.nr;  // the shared expert's group
  const int KD = STAGE == 0 ? g.H : (sh ? g.Is : g.I);
  const int NCOLS = STAGE == 0 ? (sh ? g.Is : g.I) : g.H;
  const int NT = NCOLS / COLS;  // the group's column tiles
  const int KB = KD / 128;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 2, wn = wave & 3;
  const int n0 = tc.n_tile * COLS;

  const uint8_t *wa, *wb = nullptr;
  const float *sa_w, *sb_w = nullptr;
  if (STAGE == 0) {
    wa = static_cast<const uint8_t*>(sh ? g.sh_gate : g.w_gate[tc.expert]);
    wb = static_cast<const uint8_t*>(sh ? g.sh_up : g.w_up[tc.expert]);
    sa_w = sh ? g.sh_gate_s : g.s_gate[tc.expert];
    sb_w = sh ? g.sh_up_s : g.s_up[tc.expert];
  } else {
    wa = static_cast<const uint8_t*>(sh ? g.sh_down : g.w_down[tc.expert]);
    sa_w = sh ? g.sh_down_s : g.s_down[tc.expert];
  }
  __syncthreads();  // every wave is done with the scheduler scratch before the loads reuse it
  // weight-block scales ([NCOLS / 128, KB] grid) of the tile into LDS: gate/up: row 0 the gate
  // block, row 1 the up block of the tile's 128 columns; down: the tile's two column blocks
  if (tid < 2 * SMAXKB) {
    const int which = tid / SMAXKB, kb = tid % SMAXKB;
    if (kb < KB) {
      const float* src = STAGE == 0 ? (which == 0 ? sa_w : sb_w) + (size_t)tc.n_tile * KB
                                    : sa_w + (size_t)(2 * tc.n_tile + which) * KB;
      s_ws[which * SMAXKB + kb] = ldg_f32(src + kb);
    }
  }

  // load sources.  One 16-byte instruction writes 8 rows x 128 B; lane l covers row l / 8 of
  // its group and slot l % 8, i.e. logical chunk (l % 8) ^ swz(row), swz(row) = (row / 2) % 8.
  // A fragment read serves 16 lanes (16 consecutive rows, one chunk) per LDS cycle: with this
  // swizzle they fall in 16 different 16-byte bank groups (row % 8 left rows r and r + 8 on the
  // same banks).  Instruction i writes rows 8 i + prow past a multiple of 16, so there
  // swz = (4 i + prow / 2) % 8.
  const int prow = lane >> 3;
  auto lch = [&](int lds_row) { return (lane & 7) ^ ((lds_row >> 1) & 7); };
  auto a_row = [&](int trow) -> long {  // source row of tile row trow (clamped into the segment)
    int p = tc.row0 + trow;
    if (p >= tc.row_end) p = tc.row_end - 1;  // rows past the segment are computed, never stored
    return STAGE == 0 ? (sh ? p : g.sorted_ids[p] / g.K) : p;
  };
  const uint8_t* a_ptr[SAI];  // A: wave w fills tile rows SAR w .. SAR w + SAR - 1
#pragma unroll
  for (int i = 0; i < SAI; ++i) {
    const int r = wave * SAR + 8 * i + prow;
    a_ptr[i] = static_cast<const uint8_t*>(sh ? g.sh_a : g.a) + (size_t)a_row(r) * KD + (lch(r) << 4);
  }
  // B: wave w fills weight rows SBR w .. SBR w + SBR - 1 (gate/up: the first 128 gate, the rest up)
  const uint8_t* b_ptr[SBI];
#pragma unroll
  for (int i = 0; i < SBI; ++i) {
    const int r = wave * SBR + 8 * i + prow;
    const uint8_t* row_base = STAGE == 0 ? (r < SBNB / 2 ? wa + (size_t)(n0 + r) * KD : wb + (size_t)(n0 + r - SBNB / 2) * KD)
                                         : wa + (size_t)(n0 + r) * KD;
    b_ptr[i] = row_base + (lch(r) << 4);
  }
  // row scales: lanes 0 .. SAR - 1 of wave w load the scale of tile row SAR w + lane
  const float* sc_ptr = (sh ? g.sh_a_scales : g.a_scales) + (size_t)a_row(wave * SAR + (lane % SAR)) * KB;

  auto issue = [&](int buf, int kb) {
    uint8_t* sa = smem + buf * SSTAGE;
    uint8_t* sb = sa + SABYTES;
    uint8_t* ss = sb + SBBYTES;
    const size_t koff = (size_t)kb * SROWB;
#pragma unroll
    for (int i = 0; i < SAI; ++i) dma16(a_ptr[i] + koff, sa + (wave * SAI + i) * 1024);
#pragma unroll
    for (int i = 0; i < SBI; ++i) dma16(b_ptr[i] + koff, sb + (wave * SBI + i) * 1024);
    if (lane < SAR)
      __builtin_amdgcn_global_load_lds((dma_gptr_t)(sc_ptr + kb), (dma_lptr_t)(ss + wave * SAR * 4), 4, 0, 0);
  };
  auto lds16 = [&](const uint8_t* base, int row, int chunk) {
    return *reinterpret_cast<const u32x4*>(base + row * SROWB + ((chunk ^ ((row >> 1) & 7)) << 4));
  };

  f32x16 acc[SMI][2], blk[SMI][2];
#pragma unroll
  for (int mi = 0; mi < SMI; ++mi)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][nb][r] = 0.f;

  // 32x32x64 operands: lane l holds row l % 32 and bytes 32 (l / 32) .. +31 of the 64-byte k slice;
  // D: lane l, item r -> row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
  const int frow = lane & 31, fh = lane >> 5;
  auto item_row = [&](int r) { return 8 * (r / 4) + 4 * fh + (r % 4); };
  // weight rows of block nb: gate/up nb 0 -> gate columns 32 wn, nb 1 -> the same up columns
  // (LDS rows 128 + ...); down: 64 wn + 32 nb
  auto brow = [&](int nb) { return STAGE == 0 ? nb * 128 + wn * 32 + frow : wn * 64 + nb * 32 + frow; };
  // weight-scale row of block nb: gate/up: gate (0) or up (1); down: column block of 64 wn + 32 nb
  const int ws_row0 = STAGE == 0 ? 0 : (wn * 64) / 128, ws_row1 = STAGE == 0 ? 1 : (wn * 64 + 32) / 128;

  // 32-row MFMA blocks that lie wholly past the segment's last row hold only padding: their
  // waves skip the fragment reads and products (wave-uniform), which leaves them zero
  int live_mi = 0;
#pragma unroll
  for (int mi = 0; mi < SMI; ++mi) live_mi += tc.row0 + wm * SWR + mi * 32 < tc.row_end;

#pragma unroll
  for (int s = 0; s < SNSTAGE - 1; ++s)
    if (s < KB) issue(s, s);

  for (int kb = 0; kb < KB; ++kb) {
    if (kb + 1 < KB) dma_wait<SVM>();  // step kb has landed (one later stage may still be in flight)
    else dma_wait<0>();
    __builtin_amdgcn_s_barrier();  // ... in every wave; every wave is done with step kb - 1
    __builtin_amdgcn_sched_barrier(0);
    if (kb + SNSTAGE - 1 < KB) issue((kb + SNSTAGE - 1) % SNSTAGE, kb + SNSTAGE - 1);
    if (live_mi == 0) continue;
    const uint8_t* sa = smem + (kb % SNSTAGE) * SSTAGE;
    const uint8_t* sb = sa + SABYTES;
    const float* ss = reinterpret_cast<const float*>(sb + SBBYTES);
    // fragment reads and MFMAs at raised wave priority: a wave whose operands are ready issues ahead of
    // the waves in their scale promotions (back to normal priority before its own promotions)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {  // 64-byte k slices: logical chunks 4 ks + 2 (l / 32) and +1
      const int c0 = 4 * ks + 2 * fh;
      i32x8 af[SMI], bf[2];
#pragma unroll
      for (int mi = 0; mi < SMI; ++mi) {
        if (mi >= live_mi) continue;
        const int row = wm * SWR + mi * 32 + frow;
        const u32x4 lo = lds16(sa, row, c0), hi = lds16(sa, row, c0 + 1);
        af[mi] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const u32x4 lo = lds16(sb, brow(nb), c0), hi = lds16(sb, brow(nb), c0 + 1);
        bf[nb] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int mi = 0; mi < SMI; ++mi)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          if (mi >= live_mi) continue;
          if (ks == 0) blk[mi][nb] = mfma_32x32x64_fp8(af[mi], bf[nb], f32x16{});
          else blk[mi][nb] = mfma_32x32x64_fp8(af[mi], bf[nb], blk[mi][nb]);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    // promote this scale block: acc += blk * (row scale * weight-block scale)
    const float ws0 = s_ws[ws_row0 * SMAXKB + kb], ws1 = s_ws[ws_row1 * SMAXKB + kb];
#pragma unroll
    for (int mi = 0; mi < SMI; ++mi) {
      if (mi >= live_mi) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // items 4 q .. 4 q + 3 are 4 consecutive rows
        const f32x4 rs = *reinterpret_cast<const f32x4*>(ss + wm * SWR + mi * 32 + 8 * q + 4 * fh);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[mi][0][4 * q + j] += blk[mi][0][4 * q + j] * (rs[j] * ws0);
          acc[mi][1][4 * q + j] += blk[mi][1][4 * q + j] * (rs[j] * ws1);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  if (STAGE == 1) {
    uint16_t* out = static_cast<uint16_t*>(sh ? g.sh_out : g.out);
#pragma unroll
    for (int mi = 0; mi < SMI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tc.row0 + wm * SWR + mi * 32 + item_row(r);
        if (row >= tc.row_end) continue;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          out[(size_t)row * NCOLS + n0 + wn * 64 + nb * 32 + frow] = (uint16_t)f32_to_bf16(acc[mi][nb][r]);
      }
    return;
  }

  // gate/up epilogue: h = silu(g) * u, quantised per row over the tile's 128 columns.  The h values
  // go through LDS (the ring is free) so that each row is finished by the 8 threads that hold it:
  // an amax over 8 lanes, and the codes leave as 4-byte stores.
  __syncthreads();
  constexpr int HSTRIDE = SBNB / 2 + 4;  // floats per LDS row (4 floats of padding: the two halves of a
                                         // wave write rows 4 apart, which then fall on other banks)
  float* h_lds = reinterpret_cast<float*>(smem);  // [SBM][HSTRIDE]
#pragma unroll
  for (int mi = 0; mi < SMI; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      h_lds[(wm * SWR + mi * 32 + item_row(r)) * HSTRIDE + wn * 32 + frow] = silu(acc[mi][0][r]) * acc[mi][1][r];
  __syncthreads();
  uint8_t* out = static_cast<uint8_t*>(sh ? g.sh_out : g.out);
  float* out_scales = sh ? g.sh_out_scales : g.out_scales;
  constexpr int TPR = W::WAVES * 64 / SBM;  // threads per row (8 for 16 waves)
  constexpr int VPT = SBNB / 2 / TPR;        // values per thread
  static_assert(TPR * VPT == SBNB / 2 && VPT % 4 == 0 && (TPR & (TPR - 1)) == 0, "row split");
  const int trow = tid / TPR, seg = tid % TPR;
  // thread seg of a row holds the float4 groups at columns 4 seg + 4 TPR i: the TPR threads of a row
  // read one contiguous span per instruction
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
    if (seg == 0) out_scales[(size_t)row * NT + tc.n_tile] = amax > 0.f ? amax / 448.0f : 1.0f;
  }
}

// ---- the streaming down stage with persistent blocks, one per CU
//
// The same tiles, ring, MFMAs and promotions as k_grouped_gemm_fp8_stream<1> (so the same bits), but
// block b of XCD x = b % 8 walks the tiles b / 8, b / 8 + S, ... (S blocks per XCD) of that XCD's
// contiguous range of logical tiles, and the ring does not drain between them: at the first K step
// of a tile the block finds its next tile and starts loading that tile's weight-block scales (into
// the other of two LDS buffers), and the last two K steps issue the next tile's first two stages.
// The tile prefix is built once per block.  A down tile streams 16 K steps in ~10 us, so the
// per-tile scheduler, first-stage latency and epilogue of the one-tile-per-block kernel cost a
// large share of its time.
constexpr int P_WS_OFF = SNSTAGE * SSTAGE;                   // [2 buffers][2 column blocks][SMAXKB]
constexpr int P_PREFIX_OFF = P_WS_OFF + 2 * 2 * SMAXKB * 4;  // tile prefix + the scan's wave sums
constexpr int PLDS = P_PREFIX_OFF + (kMaxGroups + 1 + kMaxSchedWaves) * 4;
static_assert(PLDS <= 160 * 1024, "one block per CU");

// One tile of the persistent down kernel: wave-uniform place and this lane's operand addresses.
struct DownTile {
  int expert, n_tile, row0, row_end, KB, live_mi, sh;
  const uint8_t* a_ptr[StreamWaves<1>::AI];  // this lane's A chunks
  const uint8_t* b_ptr[StreamWaves<1>::BI];  // this lane's B chunks
  const float* sc_ptr;                       // this lane's row scales
};

__global__ __launch_bounds__(StreamWaves<1>::WAVES * 64, 1) void k_grouped_gemm_fp8_down_persistent(GroupedGemmArgs g) {
  using W = StreamWaves<1>;
  constexpr int SWR = W::WR, SMI = W::MI, SAR = W::AR, SAI = W::AI, SBR = W::BR, SBI = W::BI, SVM = W::VM;
  extern __shared__ __align__(16) uint8_t smem[];
  float* s_ws = reinterpret_cast<float*>(smem + P_WS_OFF);  // [buffer][column block][SMAXKB]
  int* s_prefix = reinterpret_cast<int*>(smem + P_PREFIX_OFF);
  int* s_wsum = s_prefix + kMaxGroups + 1;

  const Groups G = gemm_groups(g, 1, SBNB);
  const int T = tile_prefix(G, SBM, s_prefix, s_wsum);
  // this block's tiles: XCD x's range [x chunk, min((x + 1) chunk, T)), every S-th from b / 8
  const int S = (int)gridDim.x / 8, x = blockIdx.x % 8;
  const int chunk = (T + 7) / 8;
  const int t_end = min((x + 1) * chunk, T);
  int L = x * chunk + (int)blockIdx.x / 8;
  if (L >= t_end) return;  // the same decision in every thread

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 2, wn = wave & 3;
  const int prow = lane >> 3;
  auto lch = [&](int lds_row) { return (lane & 7) ^ ((lds_row >> 1) & 7); };

  // the place of tile Lt, and direct-to-LDS loads of its weight-block scales (the tile's two column
  // blocks: waves 2 and 3, one lane per K block) into buffer buf; a later ring wait covers the loads
  auto prepare = [&](int Lt, DownTile& t, int buf) {
    const TileCoord tc = tile_at_uniform(G, SBM, s_prefix, T, Lt, 32);
    t.expert = __builtin_amdgcn_readfirstlane(tc.expert);
    t.n_tile = __builtin_amdgcn_readfirstlane(tc.n_tile);
    t.row0 = __builtin_amdgcn_readfirstlane(tc.row0);
    t.row_end = __builtin_amdgcn_readfirstlane(tc.row_end);
    t.sh = t.expert == G.nr;
    t.KB = (t.sh ? g.Is : g.I) / 128;
    t.live_mi = 0;
#pragma unroll
    for (int mi = 0; mi < SMI; ++mi) t.live_mi += t.row0 + wm * SWR + mi * 32 < t.row_end;
    if (wave == 2 || wave == 3) {
      const int which = wave - 2, kb = lane;
      if (kb < t.KB) {
        const float* src =
            (t.sh ? g.sh_down_s : table_entry_uniform(g.s_down, t.expert)) + (size_t)(2 * t.n_tile + which) * t.KB;
        __builtin_amdgcn_global_load_lds((dma_gptr_t)(src + kb), (dma_lptr_t)(s_ws + (buf * 2 + which) * SMAXKB), 4,
                                         0, 0);
      }
    }
  };
  // this lane's operand addresses for tile t (the same as the one-tile kernel's)
  auto addresses = [&](DownTile& t) {
    const int KD = t.sh ? g.Is : g.I;
    auto a_row = [&](int trow) -> long {
      int p = t.row0 + trow;
      if (p >= t.row_end) p = t.row_end - 1;  // rows past the segment are computed, never stored
      return p;
    };
#pragma unroll
    for (int i = 0; i < SAI; ++i) {
      const int r = wave * SAR + 8 * i + prow;
      t.a_ptr[i] = static_cast<const uint8_t*>(t.sh ? g.sh_a : g.a) + (size_t)a_row(r) * KD + (lch(r) << 4);
    }
    const uint8_t* wd = static_cast<const uint8_t*>(t.sh ? g.sh_down : table_entry_uniform(g.w_down, t.expert));
#pragma unroll
    for (int i = 0; i < SBI; ++i) {
      const int r = wave * SBR + 8 * i + prow;
      t.b_ptr[i] = wd + (size_t)(t.n_tile * SBNB + r) * KD + (lch(r) << 4);
    }
    t.sc_ptr = (t.sh ? g.sh_a_scales : g.a_scales) + (size_t)a_row(wave * SAR + (lane % SAR)) * t.KB;
  };
  auto issue = [&](const DownTile& t, int slot, int kb) {
    uint8_t* sa = smem + slot * SSTAGE;
    uint8_t* sb = sa + SABYTES;
    uint8_t* ss = sb + SBBYTES;
    const size_t koff = (size_t)kb * SROWB;
#pragma unroll
    for (int i = 0; i < SAI; ++i) dma16(t.a_ptr[i] + koff, sa + (wave * SAI + i) * 1024);
#pragma unroll
    for (int i = 0; i < SBI; ++i) dma16(t.b_ptr[i] + koff, sb + (wave * SBI + i) * 1024);
    if (lane < SAR)
      __builtin_amdgcn_global_load_lds((dma_gptr_t)(t.sc_ptr + kb), (dma_lptr_t)(ss + wave * SAR * 4), 4, 0, 0);
  };
  auto lds16 = [&](const uint8_t* base, int row, int chunk) {
    return *reinterpret_cast<const u32x4*>(base + row * SROWB + ((chunk ^ ((row >> 1) & 7)) << 4));
  };
  const int frow = lane & 31, fh = lane >> 5;
  auto item_row = [&](int r) { return 8 * (r / 4) + 4 * fh + (r % 4); };
  auto brow = [&](int nb) { return wn * 64 + nb * 32 + frow; };
  const int ws_row0 = (wn * 64) / 128, ws_row1 = (wn * 64 + 32) / 128;

  // the first tile: found, its scales loaded and its first two stages issued
  DownTile cur, nxt;
  int buf = 0;
  prepare(L, cur, buf);
  addresses(cur);
  int gs = 0;  // ring stage of the current tile's K step 0
#pragma unroll
  for (int s = 0; s < SNSTAGE - 1; ++s)
    if (s < cur.KB) issue(cur, s, s);

  for (;;) {
    const int Lnext = L + S;
    const bool has_next = Lnext < t_end;
    bool cross = false;  // the next tile's first stages come from this tile's last two steps
    f32x16 acc[SMI][2], blk[SMI][2];
#pragma unroll
    for (int mi = 0; mi < SMI; ++mi)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][nb][r] = 0.f;

    for (int kb = 0; kb < cur.KB; ++kb) {
      const bool later = cross || kb + 1 < cur.KB;  // a stage was issued after this one
      if (later) dma_wait<SVM>();  // step kb has landed (the one stage after it may still be in flight)
      else dma_wait<0>();
      __builtin_amdgcn_s_barrier();  // ... in every wave; every wave is done with step kb - 1
      __builtin_amdgcn_sched_barrier(0);
      if (kb + SNSTAGE - 1 < cur.KB) {
        issue(cur, (gs + kb + SNSTAGE - 1) % SNSTAGE, kb + SNSTAGE - 1);
      } else if (cross) {
        // the next tile's K step kb + 2 - KB (its addresses taken here, not kept live through the loop)
        DownTile t = nxt;
        addresses(t);
        issue(t, (gs + kb + SNSTAGE - 1) % SNSTAGE, kb + SNSTAGE - 1 - cur.KB);
      }
      if (kb == 0 && has_next && cur.KB >= 4) {
        // after this step's issue; its scale loads are older than step 3's stage, so they have landed
        // by the wait of step 2 of ... this tile (KB >= 4), long before the next tile reads them
        prepare(Lnext, nxt, buf ^ 1);
        cross = nxt.KB >= 2;
      }
      if (cur.live_mi == 0) continue;
      const uint8_t* sa = smem + ((gs + kb) % SNSTAGE) * SSTAGE;
      const uint8_t* sb = sa + SABYTES;
      const float* ss = reinterpret_cast<const float*>(sb + SBBYTES);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c0 = 4 * ks + 2 * fh;
        i32x8 af[SMI], bf[2];
#pragma unroll
        for (int mi = 0; mi < SMI; ++mi) {
          if (mi >= cur.live_mi) continue;
          const int row = wm * SWR + mi * 32 + frow;
          const u32x4 lo = lds16(sa, row, c0), hi = lds16(sa, row, c0 + 1);
          af[mi] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const u32x4 lo = lds16(sb, brow(nb), c0), hi = lds16(sb, brow(nb), c0 + 1);
          bf[nb] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
#pragma unroll
        for (int mi = 0; mi < SMI; ++mi)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            if (mi >= cur.live_mi) continue;
            if (ks == 0) blk[mi][nb] = mfma_32x32x64_fp8(af[mi], bf[nb], f32x16{});
            else blk[mi][nb] = mfma_32x32x64_fp8(af[mi], bf[nb], blk[mi][nb]);
          }
      }
      __builtin_amdgcn_s_setprio(0);
      const float ws0 = s_ws[(buf * 2 + ws_row0) * SMAXKB + kb], ws1 = s_ws[(buf * 2 + ws_row1) * SMAXKB + kb];
#pragma unroll
      for (int mi = 0; mi < SMI; ++mi) {
        if (mi >= cur.live_mi) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 rs = *reinterpret_cast<const f32x4*>(ss + wm * SWR + mi * 32 + 8 * q + 4 * fh);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[mi][0][4 * q + j] += blk[mi][0][4 * q + j] * (rs[j] * ws0);
            acc[mi][1][4 * q + j] += blk[mi][1][4 * q + j] * (rs[j] * ws1);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    {
      uint16_t* out = static_cast<uint16_t*>(cur.sh ? g.sh_out : g.out);
      const int n0 = cur.n_tile * SBNB;
#pragma unroll
      for (int mi = 0; mi < SMI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = cur.row0 + wm * SWR + mi * 32 + item_row(r);
          if (row >= cur.row_end) continue;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            out[(size_t)row * g.H + n0 + wn * 64 + nb * 32 + frow] = (uint16_t)f32_to_bf16(acc[mi][nb][r]);
        }
    }

    if (!has_next) break;
    gs += cur.KB;
    L = Lnext;
    buf ^= 1;
    if (cross) {
      cur = nxt;
      addresses(cur);
    } else {
      // not started ahead (a short tile): find it now and issue its first stages.  Every wave is past
      // the last step's barrier, so no wave still reads the ring stages these loads overwrite... the
      // ones of steps KB - 1 and KB - 2 may be read by a slower wave: wait for all before reusing them.
      __syncthreads();
      prepare(L, cur, buf);
      addresses(cur);
#pragma unroll
      for (int s = 0; s < SNSTAGE - 1; ++s)
        if (s < cur.KB) issue(cur, (gs + s) % SNSTAGE, s);
    }
  }
}

template <int STAGE>
hipError_t launch_stream(const GroupedGemmArgs& g, hipStream_t s) {
  const unsigned grid = grouped_grid(g, gemm_groups(g, STAGE, STAGE == 0 ? SBNB / 2 : SBNB), SBM);
  if (STAGE == 1) {
    // one block per CU, a multiple of 8 (the XCDs), and no more than the tiles can use
    const int cus = device_cus();
    if (cus >= 8) {
      const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_grouped_gemm_fp8_down_persistent), PLDS);
      if (e != hipSuccess) return e;
      unsigned pgrid = (unsigned)(cus / 8 * 8);
      if (grid < pgrid) pgrid = grid;  // grouped_grid is a multiple of 8
      k_grouped_gemm_fp8_down_persistent<<<pgrid, StreamWaves<1>::WAVES * 64, PLDS, s>>>(g);
      return hipGetLastError();
    }
  }
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_grouped_gemm_fp8_stream<STAGE>), SLDS);
  if (e != hipSuccess) return e;
  k_grouped_gemm_fp8_stream<STAGE><<<grid, StreamWaves<STAGE>::WAVES * 64, SLDS, s>>>(g);
  return hipGetLastError();
}

}  // namespace

bool fp8_streams(const GroupedGemmArgs& g) {
  // up to ~256 rows per group weight streaming dominates (routed experts); the shared expert's gate/up
  // (every token, one group) also runs faster on the streaming kernel, its down stage on the
  // register-staged one once the batch passes 256 tokens.  A launch that carries both streams only
  // when each part would on its own (every group keeps the kernel, and the bits, of its own launch).
  if (g.row_invariant || (g.stage == 1 && g.H % SBNB != 0)) return false;
  auto kd_fits = [&](int I) { return (g.stage == 0 ? g.H : I) <= 128 * SMAXKB; };
  const bool routed = (long)g.P <= 256L * g.E && kd_fits(g.I);
  const bool shared = (g.stage == 0 || g.N <= 256) && kd_fits(g.Is);
  if (g.shared) return shared;
  return routed && (!g.with_shared || shared);
}

hipError_t launch_grouped_gemm_fp8(const GroupedGemmArgs& g, hipStream_t s) {
  if (g.N == 0) return hipSuccess;
  if (fp8_streams(g)) return g.stage == 0 ? launch_stream<0>(g, s) : launch_stream<1>(g, s);
  if (g.stage == 0) {
    k_grouped_gemm_fp8<0><<<grouped_grid(g, gemm_groups(g, 0, BN), BM), 256, 0, s>>>(g);
  } else {
    k_grouped_gemm_fp8<1><<<grouped_grid(g, gemm_groups(g, 1, BN), BM), 256, 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace moe
