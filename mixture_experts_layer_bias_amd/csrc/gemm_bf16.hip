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

// 16-byte global load from a base that is the same in every lane plus a per-lane byte offset: with a
// 32-bit offset the base stays in scalar registers and the address costs one VGPR.  (The empty asm keeps
// the compiler from hoisting a 64-bit form of the offset out of the K loop, which would cost two VGPRs
// and a 64-bit add per load.)
__device__ __forceinline__ u32x4 ldg16_off(const void* base, uint32_t off) {
  asm volatile("" : "+v"(off));
  return *(global_u32x4*)(reinterpret_cast<const char*>(base) + off);
}
// the same for operands of 4 GiB or more
__device__ __forceinline__ u32x4 ldg16_off(const void* base, uint64_t off) {
  return *(global_u32x4*)(reinterpret_cast<const char*>(base) + off);
}
// A pointer that is the same in every lane, moved to scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// OffT: the type of the A rows' byte offsets (uint32_t while the A operand is below 4 GiB)
template <int STAGE, typename OffT>
__global__ __launch_bounds__(256, 2) void k_grouped_gemm_bf16(GroupedGemmArgs g) {
  using T = Bf16Tile<STAGE>;
  __shared__ __align__(16) uint16_t lds[T::LDS_BYTES / 2];
  uint16_t* a_lds = lds;
  uint16_t* b_lds = lds + BM * LDS_STRIDE;
  __shared__ int s_prefix[kMaxGroups + 1];
  __shared__ int s_wsum[4];

  __shared__ int s_last;

  // ---- which tile (and which part of its K range) this block computes.  The T tiles fill `slots`
  // blocks in F = T / slots full rounds and a last round of R tiles; when that round is at most half
  // full, each of its tiles is split along K into S parts (S = slots / R, at most kSplitParts and the
  // K steps of a tile), so the last round ends after about 1 / S of a tile.  Blocks 0 .. F slots - 1
  // take the whole tiles (XCD-aware, as schedule_tile), the next R S blocks the parts.
  const Groups G = gemm_groups(g, STAGE, T::COLS);
  const int ntiles = tile_prefix(G, BM, s_prefix, s_wsum);
  int S = 1, W = 0, R = 0;
  if (g.slots > 0) {
    const int F = ntiles / g.slots;
    W = F * g.slots;
    R = ntiles - W;
    // parts: at most the K steps of the shortest group (gate/up: H; down: I, and Is with the shared group)
    const int kmin = STAGE == 0 ? g.H : (g.shared ? g.Is : ((g.with_shared && g.Is < g.I) ? g.Is : g.I));
    if (R > 0) S = min(min(g.slots / R, kSplitParts), kmin / BK);
  }
  int part = -1, L;
  const int b = blockIdx.x;
  if (S >= 2) {
    if (b < W) {
      L = (b % 8) * (W / 8) + b / 8;
    } else {
      const int u = b - W;
      if (u >= R * S) return;  // the same decision in every thread
      L = W + u / S;
      part = u % S;
    }
  } else {
    const int chunk = (ntiles + 7) / 8;
    L = (b % 8) * chunk + b / 8;
    if (b / 8 >= chunk || L >= ntiles) return;
  }
  const TileCoord tc = tile_at(G, BM, s_prefix, ntiles, L);
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
  const uint16_t* a_src = uniform_ptr(static_cast<const uint16_t*>(sh ? g.sh_a : g.a));
  wa = uniform_ptr(wa);
  if (STAGE == 0) wb = uniform_ptr(wb);
  const int n0u = __builtin_amdgcn_readfirstlane(n0);

  const int lrow = tid >> 3;       // 0..31: row within a 32-row slab of the tile
  const int lcol = (tid & 7) * 8;  // bf16 column of this thread's 16-byte chunk
  // A rows: byte offsets from a_src
  OffT a_off[T::A_LOADS];
#pragma unroll
  for (int i = 0; i < T::A_LOADS; ++i) {
    int p = tc.row0 + lrow + 32 * i;
    if (p >= tc.row_end) p = tc.row_end - 1;  // clamp: rows past the segment are computed, never stored
    int arow;
    if (STAGE == 0) arow = sh ? p : g.sorted_ids[p] / g.K;
    else arow = p;
    a_off[i] = ((OffT)arow * (OffT)KD + (OffT)lcol) * 2u;
  }
  // B rows: slab i of 32 weight rows starts at a uniform address; every slab has the same per-lane offset
  const uint16_t* b_slab[T::B_LOADS];
#pragma unroll
  for (int i = 0; i < T::B_LOADS; ++i) {
    if (STAGE == 0) {
      b_slab[i] = i < T::B_LOADS / 2 ? wa + (size_t)(n0u + 32 * i) * KD : wb + (size_t)(n0u + 32 * i - BN) * KD;
    } else {
      b_slab[i] = wa + (size_t)(n0u + 32 * i) * KD;
    }
  }
  const uint32_t b_off = ((uint32_t)lrow * (uint32_t)KD + lcol) * 2u;

  u32x4 ra[T::A_LOADS], rb[T::B_LOADS];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) ra[i] = ldg16_off(a_src + k0, a_off[i]);
#pragma unroll
    for (int i = 0; i < T::B_LOADS; ++i) rb[i] = ldg16_off(b_slab[i] + k0, b_off);
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

  const int nk_all = KD / BK;
  // K steps [kt0, nk) of this block: all of them, or part `part` of S
  const int kt0 = part < 0 ? 0 : part * nk_all / S;
  const int nk = part < 0 ? nk_all : (part + 1) * nk_all / S;
  load_tile(kt0 * BK);
  store_tile();
  __syncthreads();
  for (int kt = kt0; kt < nk; ++kt) {
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

  // ---- a part of a split tile: store its partial sums (at device scope, past the per-XCD L2s), count
  // itself, and leave unless it is the last part of its tile to arrive; that one adds the S partial
  // sums in part order, its own read back like the others' (the same sums whichever part arrives
  // last), and runs the epilogue.
  if (part >= 0) {
    const int tile = L - W;  // the split tile's index, 0 .. R - 1
    float* const mine = g.split_part + (size_t)(tile * S + part) * kSplitFloats;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __hip_atomic_store(mine + ((mi * NB + nb) * 16 + r) * 256 + tid, acc[mi][nb][r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);  // the stores are complete
    __syncthreads();
    if (tid == 0) {
      // count this part: the word is (split_seq, parts arrived), or anything else before the first part
      unsigned long long* const w = g.split_cnt + tile;
      const unsigned long long tag = (unsigned long long)g.split_seq << 32;
      unsigned long long old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), nw;
      do {
        nw = (old & 0xFFFFFFFF00000000ull) == tag ? old + 1 : tag + 1;
      } while (!__hip_atomic_compare_exchange_strong(w, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT));
      s_last = (int)(nw & 0xFFFFFFFFu) == S;
      if (s_last) __hip_atomic_store(w, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    // 16 accumulators at a time: every part's 16 values are loaded before the first add, so a group
    // costs one memory round trip (parts past S reload part S - 1 and add nothing)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float v[kSplitParts][16];
#pragma unroll
        for (int q = 0; q < kSplitParts; ++q) {
          const float* src = g.split_part + (size_t)(tile * S + min(q, S - 1)) * kSplitFloats +
                             (mi * NB + nb) * 16 * 256 + tid;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            v[q][r] = __hip_atomic_load(src + r * 256, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sum = 0.f;
#pragma unroll
          for (int q = 0; q < kSplitParts; ++q)
            if (q < S) sum += v[q][r];
          acc[mi][nb][r] = sum;
        }
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

// ---- the same tiles with persistent blocks (launches that split no tile)
//
// Block b of XCD x = b % 8 walks the tiles b / 8, b / 8 + S, ... (S blocks per XCD) of that XCD's
// contiguous range of logical tiles, two blocks per CU as before.  The tile prefix is built once; a tile's
// last K step loads (into registers, then LDS, as every step does) the next tile's first step, so the
// operand stream does not pause for a scheduler prologue between tiles.  The next tile's place and weight
// pointers come from scalar loads and its gathered A rows' ids are loaded at the current tile's first
// step, so none of them makes the K loop wait.  Every tile's arithmetic is the one-tile kernel's (same
// bits).
template <int STAGE, typename OffT>
__global__ __launch_bounds__(256, 2) void k_grouped_gemm_bf16_persistent(GroupedGemmArgs g) {
  using T = Bf16Tile<STAGE>;
  __shared__ __align__(16) uint16_t lds[T::LDS_BYTES / 2];
  uint16_t* a_lds = lds;
  uint16_t* b_lds = lds + BM * LDS_STRIDE;
  __shared__ int s_prefix[kMaxGroups + 1];
  __shared__ int s_wsum[4];

  const Groups G = gemm_groups(g, STAGE, T::COLS);
  const int ntiles = tile_prefix(G, BM, s_prefix, s_wsum);
  const int SB = (int)gridDim.x / 8, x = blockIdx.x % 8;
  const int chunk = (ntiles + 7) / 8;
  const int t_end = min((x + 1) * chunk, ntiles);
  int L = x * chunk + (int)blockIdx.x / 8;
  if (L >= t_end) return;  // the same decision in every thread

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int lrow = tid >> 3;       // 0..31: row within a 32-row slab of the tile
  const int lcol = (tid & 7) * 8;  // bf16 column of this thread's 16-byte chunk
  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 31, fk = (lane >> 5) * 8;
  constexpr int NB = STAGE == 1 ? 2 : 4;

  // one tile's place, operands and this thread's A row ids / offsets
  struct Tile {
    int expert, n0, row0, row_end, KD, NCOLS, live_mi, sh;
    const uint16_t* a_src;
    const uint16_t* wa;
    const uint16_t* wb;
    int arow[T::A_LOADS];  // gate/up: sorted ids (then divided by K); down: sorted rows
    OffT a_off[T::A_LOADS];  // byte offsets of this thread's A rows from a_src (set by `offsets`)
  };
  // the place and pointers of tile Lt, and the loads of its A row ids (not waited for here)
  auto locate = [&](int Lt, Tile& t) {
    const TileCoord tc = tile_at_uniform(G, BM, s_prefix, ntiles, Lt);
    t.expert = tc.expert;
    t.sh = tc.expert == G.nr;
    t.row0 = tc.row0;
    t.row_end = tc.row_end;
    t.n0 = tc.n_tile * T::COLS;
    t.KD = STAGE == 0 ? g.H : (t.sh ? g.Is : g.I);
    t.NCOLS = STAGE == 0 ? (t.sh ? g.Is : g.I) : g.H;
    if (STAGE == 0) {
      t.wa = static_cast<const uint16_t*>(t.sh ? g.sh_gate : table_entry_uniform(g.w_gate, t.expert));
      t.wb = static_cast<const uint16_t*>(t.sh ? g.sh_up : table_entry_uniform(g.w_up, t.expert));
    } else {
      t.wa = static_cast<const uint16_t*>(t.sh ? g.sh_down : table_entry_uniform(g.w_down, t.expert));
      t.wb = nullptr;
    }
    t.a_src = static_cast<const uint16_t*>(t.sh ? g.sh_a : g.a);
    t.live_mi = (t.row0 + wm * 64 < t.row_end) + (t.row0 + wm * 64 + 32 < t.row_end);
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) {
      int p = t.row0 + lrow + 32 * i;
      if (p >= t.row_end) p = t.row_end - 1;  // clamp: rows past the segment are computed, never stored
      t.arow[i] = (STAGE == 0 && !t.sh) ? g.sorted_ids[p] : p;
    }
  };
  // the A rows' byte offsets, once the row ids have arrived
  auto offsets = [&](Tile& t) {
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) {
      const int arow = (STAGE == 0 && !t.sh) ? t.arow[i] / g.K : t.arow[i];
      t.a_off[i] = ((OffT)arow * (OffT)t.KD + (OffT)lcol) * 2u;
    }
  };
  u32x4 ra[T::A_LOADS], rb[T::B_LOADS];
  auto load_tile = [&](const Tile& t, int k0) {
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) ra[i] = ldg16_off(t.a_src + k0, t.a_off[i]);
    const uint32_t b_off = ((uint32_t)lrow * (uint32_t)t.KD + lcol) * 2u;
#pragma unroll
    for (int i = 0; i < T::B_LOADS; ++i) {
      const uint16_t* slab = STAGE == 0 ? (i < T::B_LOADS / 2 ? t.wa + (size_t)(t.n0 + 32 * i) * t.KD
                                                              : t.wb + (size_t)(t.n0 + 32 * i - BN) * t.KD)
                                        : t.wa + (size_t)(t.n0 + 32 * i) * t.KD;
      rb[i] = ldg16_off(uniform_ptr(slab) + k0, b_off);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) st16(a_lds + (lrow + 32 * i) * LDS_STRIDE + lcol, ra[i]);
#pragma unroll
    for (int i = 0; i < T::B_LOADS; ++i) st16(b_lds + (lrow + 32 * i) * LDS_STRIDE + lcol, rb[i]);
  };

  Tile cur, nxt;
  locate(L, cur);
  offsets(cur);
  load_tile(cur, 0);
  store_tile();
  __syncthreads();
  for (;;) {
    const int Lnext = L + SB;
    const bool has_next = Lnext < t_end;
    f32x16 acc[2][NB];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][nb][r] = 0.f;
    const int nk = cur.KD / BK;
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) {
        load_tile(cur, (kt + 1) * BK);
      } else if (has_next) {  // the next tile's first step (located at step 0: KD >= 128 gives nk >= 2)
        offsets(nxt);
        load_tile(nxt, 0);
      }
      if (kt == 0 && has_next) locate(Lnext, nxt);  // after this step's loads: its id loads queue behind them
#pragma unroll
      for (int kk = 0; kk < BK; kk += 16) {
        if (cur.live_mi == 0) break;
        u32x4 af[2], bfr[NB];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          if (mi < cur.live_mi) af[mi] = ld16(a_lds + (wm * 64 + mi * 32 + frow) * LDS_STRIDE + kk + fk);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int brow = (STAGE != 1 && nb >= 2 ? BN : 0) + wn * 64 + (nb & 1) * 32 + frow;
          bfr[nb] = ld16(b_lds + brow * LDS_STRIDE + kk + fk);
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          if (mi >= cur.live_mi) continue;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[mi][nb] = mfma_32x32x16_bf16(af[mi], bfr[nb], acc[mi][nb]);
        }
      }
      __syncthreads();
      if (kt + 1 < nk || has_next) {
        store_tile();
        __syncthreads();
      }
    }
    // epilogue (registers only: LDS may already hold the next tile's first step)
    uint16_t* out = static_cast<uint16_t*>(cur.sh ? g.sh_out : g.out);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = cur.row0 + wm * 64 + mi * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
        if (row >= cur.row_end) continue;
#pragma unroll
        for (int ni = 0; ni < (STAGE == 2 ? 4 : 2); ++ni) {
          const int col = cur.n0 + (ni >= 2 ? BN : 0) + wn * 64 + (ni & 1) * 32 + (lane % 32);
          float v;
          if (STAGE == 0) v = silu(acc[mi][ni][r]) * acc[mi][ni + 2][r];
          else v = acc[mi][ni][r];
          out[(size_t)row * cur.NCOLS + col] = (uint16_t)f32_to_bf16(v);
        }
      }
    if (!has_next) break;
    L = Lnext;
    cur = nxt;
  }
}

}  // namespace

// Whether some A operand of the launch (x or h, and the shared group's) reaches 4 GiB, so that its row
// offsets need 64 bits.
static bool a_is_wide(const GroupedGemmArgs& g) {
  const uint64_t lim = (uint64_t)1 << 32;
  if (g.stage == 0) return (uint64_t)g.N * g.H * 2 >= lim;
  const uint64_t routed = g.shared ? 0 : (uint64_t)g.P * g.I * 2;
  const uint64_t sh = (g.shared || g.with_shared) ? (uint64_t)g.N * g.Is * 2 : 0;
  return routed >= lim || sh >= lim;
}

template <int STAGE>
static void launch_stage(const GroupedGemmArgs& g, int cols, hipStream_t s) {
  const unsigned tiles = grouped_grid(g, gemm_groups(g, STAGE == 0 ? 0 : 1, cols), BM);  // a multiple of 8
  const int cus = device_cus();
  const int kd = STAGE == 0 ? g.H : (g.shared ? g.Is : g.I);
  if (g.slots <= 0 && kd <= 16 * BK && cus >= 8) {
    // short tiles and no split: persistent blocks, two per CU, a multiple of 8 (the XCDs), no more than
    // the tiles can use.  (Measured on the Zipf prefill layer: the down stage, 12 K steps, 178.9 -> 173.9
    // us; the gate/up, 32 steps, 301.6 -> 313.8 us, where the static walk balances tiles of unequal
    // length worse than the hardware's dispatch.)
    unsigned grid = (unsigned)(2 * cus / 8 * 8);
    if (tiles < grid) grid = tiles;
    if (a_is_wide(g)) k_grouped_gemm_bf16_persistent<STAGE, uint64_t><<<grid, 256, 0, s>>>(g);
    else k_grouped_gemm_bf16_persistent<STAGE, uint32_t><<<grid, 256, 0, s>>>(g);
    return;
  }
  // a split adds at most `slots` blocks (the parts of the last round's tiles) to the tiles' blocks
  const dim3 grid(tiles + (g.slots > 0 ? g.slots : 0));
  if (a_is_wide(g)) k_grouped_gemm_bf16<STAGE, uint64_t><<<grid, 256, 0, s>>>(g);
  else k_grouped_gemm_bf16<STAGE, uint32_t><<<grid, 256, 0, s>>>(g);
}

hipError_t launch_grouped_gemm_bf16(const GroupedGemmArgs& g, hipStream_t s) {
  if (g.N == 0) return hipSuccess;
  if (!g.row_invariant && decode_gemm_fits(g)) return launch_grouped_gemm_decode(g, s);
  if (g.stage == 0) launch_stage<0>(g, BN, s);
  else if (g.H % (2 * BN) == 0) launch_stage<2>(g, 2 * BN, s);
  else launch_stage<1>(g, BN, s);
  return hipGetLastError();
}

}  // namespace moe
