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
// (global_load_lds_dwordx4, 16 bytes per lane) of whole row segments, three K
// steps of loads ahead of the MFMAs, and two blocks per CU (the ring is
// the block's only LDS; the tile scheduler's scratch and the epilogue's partial
// sums are aliased onto it).  Weight rows are read in 256-byte segments where K
// is long (gate/up) and 128-byte ones where it is short (down); a probe of this
// access pattern streams equally fast at 128 to 1024 bytes per segment, so the
// segment length is chosen for the ring's depth.  Chunk c of LDS row r is stored at 16-byte slot c ^ (r % (segment / 16)),
// since the loads write rows unpadded in lane order.
//
// Waits are explicit (vmcnt of this wave's own loads, then a plain s_barrier):
// a __syncthreads would wait for every stage still in flight.
#include "common.h"
#include "dma.h"
#include "gemm_common.h"
#include "kernels.h"
#include "unpermute.h"

namespace moe {

namespace {

// Tile shapes.  A stage holds BM x ROWB bytes of A (AI load instructions per wave) and
// BNB x ROWB bytes of B (BI per wave); NSTAGE stages make the ring.
//   gate/up (K = H, long): 16 rows x 64 weight rows (32 gate, 32 up) x 256-byte segments,
//     4 x 20 KB stages (three K steps of loads ahead: the stream needs about 64 KB in flight per
//     CU, and a tile spends a few microseconds in its scheduler and epilogue with none); wave w
//     computes 32-wide k slice w of every step for the whole tile (partial sums added in the
//     epilogue).
//   down (K = I, short):   32 rows x 128 weight rows x 128-byte segments, 4 x 20 KB stages (half
//     as many tiles, so a decode layer's down tiles are all resident at once); wave w owns weight
//     rows 32w .. 32w+31.
// Both rings fit twice in a CU's LDS (two blocks per CU).
template <int STAGE>
struct DecodeShape;
template <>
struct DecodeShape<0> {
  static constexpr int BM = 16, BNB = 64, ROWB = 256, WK = 4, NSTAGE = 4, AI = 1, BI = 4;
};
template <>
struct DecodeShape<1> {
  static constexpr int BM = 32, BNB = 128, ROWB = 128, WK = 1, NSTAGE = 4, AI = 1, BI = 4;
};
template <int STAGE>
constexpr int dc_stage_bytes() {
  return (DecodeShape<STAGE>::BM + DecodeShape<STAGE>::BNB) * DecodeShape<STAGE>::ROWB;
}
template <int STAGE>
constexpr int dc_ring_bytes() {
  return DecodeShape<STAGE>::NSTAGE * dc_stage_bytes<STAGE>();
}
constexpr int DC_LDS = dc_ring_bytes<0>() > dc_ring_bytes<1>() ? dc_ring_bytes<0>() : dc_ring_bytes<1>();
static_assert(2 * DC_LDS <= 160 * 1024, "two blocks per CU");

// wait until at most `stages_after` later stages (VM loads each) are still in flight
template <int NSTAGE, int VM>
__device__ __forceinline__ void wait_stages(int stages_after) {
  static_assert(NSTAGE >= 2 && NSTAGE <= 7, "one case per possible count of later stages");
  switch (stages_after) {
    case 0: dma_wait<0>(); break;
    case 1: dma_wait<VM>(); break;
    case 2: dma_wait<(NSTAGE > 3 ? 2 * VM : VM)>(); break;
    case 3: dma_wait<(NSTAGE > 4 ? 3 * VM : VM)>(); break;
    case 4: dma_wait<(NSTAGE > 5 ? 4 * VM : VM)>(); break;
    default: dma_wait<(NSTAGE > 6 ? 5 * VM : VM)>(); break;
  }
}

__device__ __forceinline__ float silu_d(float g) { return g / (1.0f + __expf(-g)); }

// Bounded wait of a down tile for its expert's gate/up tiles (the fused launch).  The bound only
// guarantees that every wave exits; gate/up tiles never wait, and all of them are dispatched
// before the first down tile, so the count is reached long before it.  Should the bound ever be
// reached, the tile sets the error word sync[kSyncError] (which the launch never clears) and
// carries on, so that every counter still completes and is reset; that launch's output is then
// undefined and the word says so.
constexpr int kDoneSpinLimit = 1 << 22;
static_assert(kSyncExperts + kMaxGroups <= kSyncColTiles && kSyncColTiles + kSyncMaxColTiles <= kSyncReduced &&
                  kSyncReduced < kSyncError && kSyncError < kSyncInts,
              "the counters' pieces do not overlap");

// 16 bytes of y (8 bf16) at device scope: y is written in the same launch by down tiles that may
// run on other XCDs, whose L2s are not coherent with this one's
__device__ __forceinline__ u32x4 ld16_device_scope(const uint16_t* p) {
  const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __hip_atomic_load(q + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}

// The unpermute-reduce of output columns [c0, c0 + ncols) for every token, once every down tile
// of those columns is complete: the same sums, in the same order, as the unpermute-reduce
// kernel.  Slots are taken 8 at a time (loads of a batch in flight together, adds in slot order).
// With a shared-expert gate the tokens' shared weights are computed first into s_w (LDS, N
// floats).  Called by every thread of the block.
__device__ void reduce_columns(const ReduceArgs& r, const uint16_t* y, int c0, int ncols, float* s_w) {
  const int chunks = ncols / 8;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const bool gated = r.shared_y && r.shared_gate;  // the same in every thread
  if (gated) {
    __syncthreads();  // the caller's last LDS reads are done before s_w is written
    const int nw = blockDim.x / kWave, wv = threadIdx.x / kWave;
    for (int t = wv; t < r.N; t += nw) {
      const float g = shared_gate_weight(r.x + (size_t)t * r.H, r.shared_gate, r.H);
      if (threadIdx.x % kWave == 0) s_w[t] = g;
    }
    __syncthreads();
  }
  for (int p = threadIdx.x; p < r.N * chunks; p += blockDim.x) {
    const int t = p / chunks, c = c0 + (p % chunks) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float zero = 0.f;
    for (int k0 = 0; k0 < r.K; k0 += 8) {
      int rows[8];
      float wk[8];
      u32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = k0 + j;
        rows[j] = -2;  // past K
        wk[j] = 0.f;
        if (k < r.K) {
          const size_t tk = (size_t)t * r.K + k;
          rows[j] = r.ids[tk] < r.E ? r.inv_perm[tk] : -1;
          wk[j] = r.w[tk];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = rows[j] >= 0 ? ld16_device_scope(y + (size_t)rows[j] * r.H + c) : z4;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (rows[j] >= 0) acc_bf16x8(acc, wk[j], v[j]);
        else if (rows[j] == -1) zero += wk[j];
      }
    }
    const size_t xo = (size_t)t * r.H + c;
    const u32x4 xv = zero != 0.f ? ld16(r.x + xo) : z4;
    // the shared expert's y may come from down tiles of this very launch (other XCDs): device scope
    const u32x4 sv = r.shared_y ? ld16_device_scope(r.shared_y + xo) : z4;
    st16(r.out + xo, finish_bf16x8(acc, zero, xv, r.shared_y != nullptr, sv, gated ? s_w[t] : 1.0f));
  }
}

// One tile of a decode-shaped grouped GEMM.  `block` is the tile slot (blockIdx.x of a plain
// launch).  FUSED (gate/up, down and the reduce in one launch; `done` is the kSyncInts counters:
// per-expert counts at kSyncExperts, one count per down column tile at kSyncColTiles and the count
// of reduced column tiles at kSyncReduced, all zero at the start):
//   - a gate/up tile writes h with device-scope stores, waits until they are complete, then adds
//     one to its expert's count;
//   - a down tile waits until its expert's gate/up tiles are all counted, loads h at device scope,
//     writes y with device-scope stores, waits for them and adds one to its column tile's count;
//     the tile that brings that count to the number of row tiles reduces those columns, then
//     counts them; the last to do so finds every other tile finished and zeroes all the counts
//     for the next launch.
// No cache-wide write-back or invalidate is needed on either side.
template <int STAGE, bool FUSED>
__device__ __forceinline__ void decode_tile(const GroupedGemmArgs& g, uint8_t* smem, int block, int32_t* done,
                                            int gu_nt, int gu_xnt, const ReduceArgs* ra) {
  using S = DecodeShape<STAGE>;
  constexpr int BM = S::BM, BNB = S::BNB, ROWB = S::ROWB, WK = S::WK, WN = 4 / WK;
  constexpr int NSTAGE = S::NSTAGE, AI = S::AI, BI = S::BI, VM = AI + BI;
  constexpr int SBYTES = dc_stage_bytes<STAGE>();
  constexpr int ABYTES = BM * ROWB;
  constexpr int LPR = ROWB / 16;          // lanes per row in one load instruction
  constexpr int RPI = 64 / LPR;           // rows per load instruction
  constexpr int NSUB = ROWB / 64;         // 32-wide k slices per K step
  constexpr int MT = BM / 16;             // 16-row MFMA blocks
  constexpr int NTW = BNB / WN / 16;      // 16-wide weight blocks per wave
  constexpr int SUBW = NSUB / WK;         // k slices per wave per step
  static_assert(ABYTES == AI * 4 * 1024 && BNB * ROWB == BI * 4 * 1024, "one 1 KB load per wave instruction");
  static_assert(WK == 1 || 4 * BNB * BM * 4 <= NSTAGE * SBYTES, "epilogue partial sums fit in the ring");

  int* s_prefix = reinterpret_cast<int*>(smem);     // scheduler scratch, dead before the first load
  int* s_wsum = s_prefix + kMaxGroups + 1;

  const int COLS_PER_TILE = STAGE == 0 ? BNB / 2 : BNB;
  const Groups G = gemm_groups(g, STAGE, COLS_PER_TILE);
  const TileCoord tc = schedule_tile_at(G, BM, s_prefix, s_wsum, block);
  const int NT = G.nt;  // column tiles of a routed group (down: of every group)
  const bool sh = tc.expert == G.nr;  // the shared expert's group
  const int KD = STAGE == 0 ? g.H : (sh ? g.Is : g.I);
  const int NCOLS = STAGE == 0 ? (sh ? g.Is : g.I) : g.H;
  if (tc.expert < 0) {  // the same decision in every thread of the block
    // FUSED with no routed rows at all (every slot took an identity expert): no down tile counts,
    // so the first NT slots reduce one column tile each
    if (STAGE == 1 && FUSED && tc.m_tiles == 0 && block < NT)
      reduce_columns(*ra, nullptr, block * BNB, BNB, reinterpret_cast<float*>(smem) + kMaxGroups + 16);
    return;
  }
  __syncthreads();               // every wave is done with the scheduler scratch before the loads reuse it

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n0 = tc.n_tile * COLS_PER_TILE;
  const size_t row_bytes = (size_t)KD * 2;
  const int nk = KD / (ROWB / 2);

  const uint8_t *wa, *wb = nullptr;
  if (STAGE == 0) {
    wa = static_cast<const uint8_t*>(sh ? g.sh_gate : g.w_gate[tc.expert]);
    wb = static_cast<const uint8_t*>(sh ? g.sh_up : g.w_up[tc.expert]);
  } else {
    wa = static_cast<const uint8_t*>(sh ? g.sh_down : g.w_down[tc.expert]);
  }

  // Load sources.  One instruction writes RPI rows x ROWB bytes; lane l covers row l / LPR
  // of its group and 16-byte slot l % LPR, i.e. logical chunk (l % LPR) ^ (row % LPR).
  // A: instruction i of wave w fills tile rows RPI (AI w + i) ..; B: instruction i of wave w
  // fills weight rows RPI (BI w + i) .. (gate/up: the first BNB / 2 rows gate, the rest up).
  const int prow = lane / LPR, pslot = lane % LPR;
  const uint8_t* a_ptr[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int trow = (wave * AI + i) * RPI + prow;
    int p = tc.row0 + trow;
    if (p >= tc.row_end) p = tc.row_end - 1;  // rows past the segment are computed, never stored
    long arow;
    if (STAGE == 0) arow = sh ? p : g.sorted_ids[p] / g.K;
    else arow = p;
    a_ptr[i] = static_cast<const uint8_t*>(sh ? g.sh_a : g.a) + (size_t)arow * row_bytes +
               ((pslot ^ (trow % LPR)) << 4);
  }
  const uint8_t* b_ptr[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int trow = (wave * BI + i) * RPI + prow;
    const uint8_t* base;
    if (STAGE == 0)
      base = trow < BNB / 2 ? wa + (size_t)(n0 + trow) * row_bytes : wb + (size_t)(n0 + trow - BNB / 2) * row_bytes;
    else
      base = wa + (size_t)(n0 + trow) * row_bytes;
    b_ptr[i] = base + ((pslot ^ (trow % LPR)) << 4);
  }
  auto issue_a = [&](int stage, int kstep) {
    uint8_t* sa = smem + stage * SBYTES;
    const size_t koff = (size_t)kstep * ROWB;
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      if (STAGE == 1 && FUSED) dma16_device_scope(a_ptr[i] + koff, sa + (wave * AI + i) * 1024);
      else dma16(a_ptr[i] + koff, sa + (wave * AI + i) * 1024);
    }
  };
  auto issue_b = [&](int stage, int kstep) {
    uint8_t* sb = smem + stage * SBYTES + ABYTES;
    const size_t koff = (size_t)kstep * ROWB;
#pragma unroll
    for (int i = 0; i < BI; ++i) dma16(b_ptr[i] + koff, sb + (wave * BI + i) * 1024);
  };
  auto issue = [&](int stage, int kstep) {
    issue_a(stage, kstep);
    issue_b(stage, kstep);
  };
  auto lds_chunk = [&](const uint8_t* base, int row, int chunk) {
    return *reinterpret_cast<const u32x4*>(base + row * ROWB + ((chunk ^ (row % LPR)) << 4));
  };

  // this wave's weight blocks and k slices
  const int wn = wave % WN, wk = wave / WN;
  auto wrow0 = [&](int j) {  // first weight row of block j
    if (STAGE == 0) {
      const int half = j / (NTW / 2), idx = j % (NTW / 2);  // gate blocks, then the matching up blocks
      return half * (BNB / 2) + wn * (BNB / 2 / WN) + idx * 16;
    }
    return wn * (BNB / WN) + j * 16;
  };
  // 16x16x32 operands: lane l holds row l % 16, 8-element chunk 4 s + l / 16 of k slice s
  const int frow = lane & 15, fq = lane >> 4;
  f32x4 acc[MT][NTW];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[mi][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (STAGE == 1 && FUSED) {
    // The first stages' weight rows do not depend on h: they are in flight while thread 0 waits
    // for the expert's gate/up tiles, and only the h loads follow the wait.  The raw barrier
    // (no vmcnt drain) keeps those weight loads in flight.
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
      if (s < nk) issue_b(s, s);
    if (threadIdx.x == 0) {
      // the group's gate/up tiles: its row tiles times its gate/up column tiles (the shared expert's
      // intermediate size may differ from the routed experts')
      const int count = group_rows(G, tc.expert);
      const int need = (sh ? gu_xnt : gu_nt) * ((count + DecodeShape<0>::BM - 1) / DecodeShape<0>::BM);
      bool ready = false;
      for (int it = 0; it < kDoneSpinLimit && !ready; ++it) {
        ready = __hip_atomic_load(done + kSyncExperts + tc.expert, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                need;
        if (!ready) __builtin_amdgcn_s_sleep(2);
      }
      if (!ready) __hip_atomic_store(done + kSyncError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
      if (s < nk) issue_a(s, s);
  } else {
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
      if (s < nk) issue(s, s);
  }

  for (int k = 0; k < nk; ++k) {
    const int later = nk - 1 - k;  // stages issued after step k (capped by the ring depth)
    // the fused down prologue issued its stages out of order (weights, then h): the first step
    // waits for all of them
    if (STAGE == 1 && FUSED && k == 0) dma_wait<0>();
    else wait_stages<NSTAGE, VM>(later < NSTAGE - 2 ? later : NSTAGE - 2);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (k + NSTAGE - 1 < nk) issue((k + NSTAGE - 1) % NSTAGE, k + NSTAGE - 1);
    const uint8_t* sa = smem + (k % NSTAGE) * SBYTES;
    const uint8_t* sb = sa + ABYTES;
#pragma unroll
    for (int u = 0; u < SUBW; ++u) {
      const int ch = 4 * (wk * SUBW + u) + fq;
      u32x4 b[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) b[j] = lds_chunk(sb, wrow0(j) + frow, ch);
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const u32x4 a = lds_chunk(sa, mi * 16 + frow, ch);
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[mi][j] = mfma_16x16x32_bf16(a, b[j], acc[mi][j]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // epilogue.  16x16 D layout: lane l, item r -> row 16 mi + 4 (l / 16) + r, column l % 16 of the block
  uint16_t* out = static_cast<uint16_t*>(sh ? g.sh_out : g.out);
  if (WK == 1) {  // every wave holds whole sums for its weight blocks
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = tc.row0 + mi * 16 + 4 * fq + r;
        if (row >= tc.row_end) continue;
        if (STAGE == 0) {
#pragma unroll
          for (int idx = 0; idx < NTW / 2; ++idx) {
            const int col = n0 + wn * (BNB / 2 / WN) + idx * 16 + frow;
            out[(size_t)row * NCOLS + col] =
                (uint16_t)f32_to_bf16(silu_d(acc[mi][idx][r]) * acc[mi][NTW / 2 + idx][r]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            const int col = n0 + wn * (BNB / WN) + j * 16 + frow;
            uint16_t* dst = out + (size_t)row * NCOLS + col;
            if (FUSED) __hip_atomic_store(dst, (uint16_t)f32_to_bf16(acc[mi][j][r]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else *dst = (uint16_t)f32_to_bf16(acc[mi][j][r]);
          }
        }
      }
  } else {  // WN == 1: the waves' partial sums meet in LDS and are added in wave order
    __syncthreads();  // the ring is free once every wave is past its last read
    float* part = reinterpret_cast<float*>(smem);  // [wave][tile row][weight row]
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[(wave * BM + mi * 16 + 4 * fq + r) * BNB + j * 16 + frow] = acc[mi][j][r];
    __syncthreads();
    auto sum4 = [&](int row, int wr) {
      float v = part[row * BNB + wr];
#pragma unroll
      for (int w = 1; w < 4; ++w) v += part[(w * BM + row) * BNB + wr];
      return v;
    };
    constexpr int OC = STAGE == 0 ? BNB / 2 : BNB;  // output columns of the tile
    for (int o = tid; o < BM * OC; o += 256) {
      const int row = o / OC, col = o % OC;
      if (tc.row0 + row >= tc.row_end) continue;
      const float v = STAGE == 0 ? silu_d(sum4(row, col)) * sum4(row, BNB / 2 + col) : sum4(row, col);
      uint16_t* dst = out + (size_t)(tc.row0 + row) * NCOLS + n0 + col;
      if (STAGE == 0 && FUSED) __hip_atomic_store(dst, (uint16_t)f32_to_bf16(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else *dst = (uint16_t)f32_to_bf16(v);
    }
  }
  if (STAGE == 0 && FUSED) {
    static_assert(STAGE != 0 || WK == 4, "the fused h stores are the partial-sum epilogue's");
    dma_wait<0>();     // this wave's device-scope h stores are complete
    __syncthreads();   // ... and every other wave's
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(done + kSyncExperts + tc.expert, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (STAGE == 1 && FUSED) {
    static_assert(STAGE != 1 || WK == 1, "the fused y stores are the whole-sum epilogue's");
    dma_wait<0>();     // this wave's device-scope y stores are complete
    __syncthreads();   // ... and every other wave's; the ring is free
    int* s_last = reinterpret_cast<int*>(smem);
    if (threadIdx.x == 0) {
      const int before =
          __hip_atomic_fetch_add(done + kSyncColTiles + tc.n_tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_last = before == tc.m_tiles - 1;
    }
    __syncthreads();
    if (*s_last) {
      // the routed rows of y (g.out), whichever group this tile belongs to
      reduce_columns(*ra, static_cast<const uint16_t*>(g.out), n0, BNB, reinterpret_cast<float*>(smem) + 16);
      if (threadIdx.x == 0) {
        const int before =
            __hip_atomic_fetch_add(done + kSyncReduced, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last[1] = before == NT - 1;
      }
      __syncthreads();
      if (s_last[1]) {  // every other tile has counted itself: clear what this launch used
        for (int i = threadIdx.x; i < G.nr + (G.xr > 0 ? 1 : 0); i += 256)  // the groups' counts
          __hip_atomic_store(done + kSyncExperts + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int i = threadIdx.x; i < NT; i += 256)
          __hip_atomic_store(done + kSyncColTiles + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (threadIdx.x == 0) __hip_atomic_store(done + kSyncReduced, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <int STAGE>
__global__ __launch_bounds__(256, 2) void k_grouped_gemm_decode(GroupedGemmArgs g) {
  extern __shared__ __align__(16) uint8_t smem[];  // dc_ring_bytes<STAGE>() bytes
  decode_tile<STAGE, false>(g, smem, blockIdx.x, nullptr, 0, 0, nullptr);
}

// gate/up, down and the reduce of the routed experts (and, with_shared, the shared expert as one more
// group) in one launch: blocks [0, gu_blocks) take gate/up tiles, the rest take down tiles, which
// wait for their group's h (gu_blocks is a multiple of 8, so a block keeps its XCD-aware tile order).
// Workgroups are dispatched in order on each XCD, so every gate/up tile is running or done before a
// down tile of the same XCD can occupy a slot, and gate/up tiles never wait: every wait ends.
__global__ __launch_bounds__(256, 2) void k_decode_fused(GroupedGemmArgs gu, GroupedGemmArgs dn, ReduceArgs r,
                                                         int gu_blocks, int32_t* done) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int gu_nt = gu.I / (DecodeShape<0>::BNB / 2), gu_xnt = gu.Is / (DecodeShape<0>::BNB / 2);
  if ((int)blockIdx.x < gu_blocks) decode_tile<0, true>(gu, smem, blockIdx.x, done, gu_nt, gu_xnt, nullptr);
  else decode_tile<1, true>(dn, smem, blockIdx.x - gu_blocks, done, gu_nt, gu_xnt, &r);
}

template <int STAGE>
hipError_t launch_decode(const GroupedGemmArgs& g, hipStream_t s) {
  constexpr int lds = dc_ring_bytes<STAGE>();
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_grouped_gemm_decode<STAGE>), lds);
  if (e != hipSuccess) return e;
  constexpr int cols = STAGE == 0 ? DecodeShape<0>::BNB / 2 : DecodeShape<1>::BNB;
  k_grouped_gemm_decode<STAGE><<<grouped_grid(g, gemm_groups(g, STAGE, cols), DecodeShape<STAGE>::BM), 256, lds, s>>>(g);
  return hipGetLastError();
}

}  // namespace

bool decode_fused_fits(int E, int H) {
  return E <= kMaxGroups && H % DecodeShape<1>::BNB == 0 && H / DecodeShape<1>::BNB <= kSyncMaxColTiles;
}

hipError_t launch_decode_fused(const GroupedGemmArgs& gu, const GroupedGemmArgs& dn, const ReduceArgs& r,
                               int32_t* done, hipStream_t s) {
  if (gu.N == 0) return hipSuccess;
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&k_decode_fused), DC_LDS);
  if (e != hipSuccess) return e;
  const unsigned gu_blocks = grouped_grid(gu, gemm_groups(gu, 0, DecodeShape<0>::BNB / 2), DecodeShape<0>::BM);
  const unsigned dn_blocks = grouped_grid(dn, gemm_groups(dn, 1, DecodeShape<1>::BNB), DecodeShape<1>::BM);
  k_decode_fused<<<gu_blocks + dn_blocks, 256, DC_LDS, s>>>(gu, dn, r, (int)gu_blocks, done);
  return hipGetLastError();
}

namespace {

// whole K steps (ROWB / 2 elements) and whole column tiles for an expert of intermediate size I
bool decode_shape_fits(int stage, int H, int I) {
  return stage == 0 ? (H % (DecodeShape<0>::ROWB / 2) == 0 && I % (DecodeShape<0>::BNB / 2) == 0)
                    : (I % (DecodeShape<1>::ROWB / 2) == 0 && H % DecodeShape<1>::BNB == 0);
}

}  // namespace

bool decode_gemm_fits(const GroupedGemmArgs& g) {
  // routed experts: about one row tile per touched expert; the shared expert: a decode-sized batch.
  // A launch that carries both takes the decode kernels only when each part would on its own, so
  // every group gets the same kernel, and the same bits, as in a launch of its own.
  const bool routed = (long)g.P <= 8L * g.E && g.P <= 512 && decode_shape_fits(g.stage, g.H, g.I);
  const bool shared = g.N <= 64 && decode_shape_fits(g.stage, g.H, g.Is);
  if (g.shared) return shared;
  return routed && (!g.with_shared || shared);
}

hipError_t launch_grouped_gemm_decode(const GroupedGemmArgs& g, hipStream_t s) {
  if (g.N == 0) return hipSuccess;
  return g.stage == 0 ? launch_decode<0>(g, s) : launch_decode<1>(g, s);
}

}  // namespace moe
