// Grouped expert GEMMs for a few rows per expert (decode), bf16, for gfx950.
//
// forward_prefill.rs page, run_routed_grouped_gemm (grouped gate/up GEMM with
// the activation, grouped down GEMM) at the row counts of single-token decode,
// where the forward.rs page's fused decode kernels stream each selected
// expert's weights once; here the same grouped data flow does that streaming.
//
// With one to a few rows per expert the layer is bound by reading the touched
// experts' weights from HBM, so the kernel is built to keep many bytes in
// flight: a 4-stage LDS ring filled by direct global -> LDS loads
// (global_load_lds_dwordx4, 16 bytes per lane, whole 128-byte row segments),
// three K steps of loads ahead of the MFMAs, and two blocks per CU (the ring is
// the block's only LDS; the tile scheduler's scratch is aliased onto it).
// Tile: 32 sorted rows x 128 weight rows (gate/up: 64 output columns of gate
// and the same 64 of up; down: 128 output columns), K step = 64 bf16.  Each wave owns all 32 rows and 32 weight rows
// (gate/up: 16 columns of gate + the same 16 of up) as 2 x 2 tiles of
// v_mfma_f32_16x16x32_bf16.  Chunk c of LDS row r is stored at chunk
// c ^ (r & 7), since the DMA writes rows unpadded in lane order.
//
// Waits are explicit (vmcnt of this wave's own loads, then a plain s_barrier):
// a __syncthreads would wait for every stage still in flight.
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int DC_BM = 32;
constexpr int DC_BNB = 128;
constexpr int DC_ROWB = 128;  // bytes per row per K step
constexpr int DC_ABYTES = DC_BM * DC_ROWB;    // 4 KB: 1 DMA instruction per wave
constexpr int DC_BBYTES = DC_BNB * DC_ROWB;   // 16 KB: 4 per wave
constexpr int DC_STAGE = DC_ABYTES + DC_BBYTES;
constexpr int DC_NSTAGE = 4;  // 80 KB: two blocks per CU, so every tile of a decode layer is resident
constexpr int DC_VM = 5;  // DMA instructions per wave per stage

typedef const void __attribute__((address_space(1)))* gptr_t;
typedef void __attribute__((address_space(3)))* lptr_t;

__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)lds_wave_base, 16, 0, 0);
}

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 0xF) | ((N >> 4) << 14));
}

// wait until at most `stages_after` later stages (DC_VM loads each) are still in flight
__device__ __forceinline__ void wait_stages(int stages_after) {
  static_assert(DC_NSTAGE == 4, "one case per possible count of later stages");
  switch (stages_after) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1 * DC_VM>(); break;
    default: wait_vm<2 * DC_VM>(); break;
  }
}

__device__ __forceinline__ u32x4 lds_chunk(const uint8_t* base, int row, int chunk) {
  return *reinterpret_cast<const u32x4*>(base + row * DC_ROWB + ((chunk ^ (row & 7)) << 4));
}

__device__ __forceinline__ float silu_d(float g) { return g / (1.0f + __expf(-g)); }

template <int STAGE>
__global__ __launch_bounds__(256, 1) void k_grouped_gemm_decode(GroupedGemmArgs g) {
  extern __shared__ __align__(16) uint8_t smem[];  // DC_NSTAGE * DC_STAGE bytes
  int* s_prefix = reinterpret_cast<int*>(smem);     // scheduler scratch, dead before the first DMA
  int* s_wsum = s_prefix + kMaxGroups + 1;

  const int KD = STAGE == 0 ? g.H : g.I;
  const int NCOLS = STAGE == 0 ? g.I : g.H;
  const int COLS_PER_TILE = STAGE == 0 ? DC_BNB / 2 : DC_BNB;
  const int NT = NCOLS / COLS_PER_TILE;
  const TileCoord tc = schedule_tile(g.offsets, g.shared ? 1 : g.E, g.shared ? g.N : -1, DC_BM, NT, s_prefix, s_wsum);
  if (tc.expert < 0) return;  // the same decision in every thread of the block
  __syncthreads();               // every wave is done with the scheduler scratch before the DMA reuses it

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n0 = tc.n_tile * COLS_PER_TILE;
  const size_t row_bytes = (size_t)KD * 2;
  const int nk = KD / 64;

  const uint8_t *wa, *wb = nullptr;
  if (STAGE == 0) {
    wa = static_cast<const uint8_t*>(g.shared ? g.sh_gate : g.w_gate[tc.expert]);
    wb = static_cast<const uint8_t*>(g.shared ? g.sh_up : g.w_up[tc.expert]);
  } else {
    wa = static_cast<const uint8_t*>(g.shared ? g.sh_down : g.w_down[tc.expert]);
  }

  // DMA sources.  A: wave w fills tile rows 8w..8w+7; B: instruction i of wave w fills
  // weight rows (4w + i) * 8 + lane / 8 (gate/up: rows 0..63 gate, 64..127 up).
  const int prow = lane >> 3, pch = lane & 7;
  const uint8_t* a_ptr;
  {
    const int trow = wave * 8 + prow;
    int p = tc.row0 + trow;
    if (p >= tc.row_end) p = tc.row_end - 1;  // rows past the segment are computed, never stored
    long arow;
    if (STAGE == 0) arow = g.shared ? p : g.sorted_ids[p] / g.K;
    else arow = p;
    a_ptr = static_cast<const uint8_t*>(g.a) + (size_t)arow * row_bytes + ((pch ^ (trow & 7)) << 4);
  }
  const uint8_t* b_ptr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int trow = (wave * 4 + i) * 8 + prow;
    const uint8_t* base;
    if (STAGE == 0) base = trow < 64 ? wa + (size_t)(n0 + trow) * row_bytes : wb + (size_t)(n0 + trow - 64) * row_bytes;
    else base = wa + (size_t)(n0 + trow) * row_bytes;
    b_ptr[i] = base + ((pch ^ (trow & 7)) << 4);
  }
  auto issue = [&](int stage, int kstep) {
    uint8_t* sa = smem + stage * DC_STAGE;
    uint8_t* sb = sa + DC_ABYTES;
    const size_t koff = (size_t)kstep * DC_ROWB;
    dma16(a_ptr + koff, sa + wave * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(b_ptr[i] + koff, sb + (wave * 4 + i) * 1024);
  };

  // weight rows of this wave's two fragments
  const int frow = lane & 15, fq = lane >> 4;  // 16x16x32 operand: row l%16, 8-element chunk l/16
  const int br0 = STAGE == 0 ? wave * 16 + frow : wave * 32 + frow;
  const int br1 = STAGE == 0 ? 64 + wave * 16 + frow : wave * 32 + 16 + frow;

  f32x4 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mi][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < DC_NSTAGE - 1; ++s)
    if (s < nk) issue(s, s);

  for (int k = 0; k < nk; ++k) {
    const int later = nk - 1 - k;  // stages issued after step k (capped by the ring depth)
    wait_stages(later < DC_NSTAGE - 2 ? later : DC_NSTAGE - 2);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (k + DC_NSTAGE - 1 < nk) issue((k + DC_NSTAGE - 1) % DC_NSTAGE, k + DC_NSTAGE - 1);
    const uint8_t* sa = smem + (k % DC_NSTAGE) * DC_STAGE;
    const uint8_t* sb = sa + DC_ABYTES;
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // 32-element k steps: logical chunk 4j + l/16
      const int ch = 4 * j + fq;
      const u32x4 b0 = lds_chunk(sb, br0, ch), b1 = lds_chunk(sb, br1, ch);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const u32x4 a = lds_chunk(sa, mi * 16 + frow, ch);
        acc[mi][0] = mfma_16x16x32_bf16(a, b0, acc[mi][0]);
        acc[mi][1] = mfma_16x16x32_bf16(a, b1, acc[mi][1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // epilogue.  16x16 D layout: lane l, item r -> row 4*(l/16) + r, column l%16
  uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = tc.row0 + mi * 16 + 4 * fq + r;
      if (row >= tc.row_end) continue;
      if (STAGE == 0) {
        const int col = n0 + wave * 16 + frow;
        out[(size_t)row * NCOLS + col] = (uint16_t)f32_to_bf16(silu_d(acc[mi][0][r]) * acc[mi][1][r]);
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = n0 + wave * 32 + nb * 16 + frow;
          out[(size_t)row * NCOLS + col] = (uint16_t)f32_to_bf16(acc[mi][nb][r]);
        }
      }
    }
}

template <int STAGE>
hipError_t launch_decode(const GroupedGemmArgs& g, int groups, int rows, int nt, hipStream_t s) {
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_grouped_gemm_decode<STAGE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, DC_NSTAGE * DC_STAGE);
    if (e != hipSuccess) return e;
    configured = true;
  }
  k_grouped_gemm_decode<STAGE><<<grouped_grid(rows, groups, DC_BM, nt), 256, DC_NSTAGE * DC_STAGE, s>>>(g);
  return hipGetLastError();
}

}  // namespace

bool decode_gemm_fits(const GroupedGemmArgs& g) {
  const int groups = g.shared ? 1 : g.E;
  const int rows = g.shared ? g.N : g.P;
  const bool few_rows = rows <= 8L * groups && rows <= 512;  // about one 32-row tile per touched expert
  return few_rows && (g.stage == 0 ? g.I % 64 == 0 : g.H % 128 == 0);
}

hipError_t launch_grouped_gemm_decode(const GroupedGemmArgs& g, hipStream_t s) {
  const int groups = g.shared ? 1 : g.E;
  const int rows = g.shared ? g.N : g.P;
  if (rows == 0) return hipSuccess;
  return g.stage == 0 ? launch_decode<0>(g, groups, rows, g.I / 64, s) : launch_decode<1>(g, groups, rows, g.H / 128, s);
}

}  // namespace moe
