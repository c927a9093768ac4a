// Device-side tile scheduler shared by the grouped expert GEMMs.
//
// The rows of each routed expert are a contiguous segment [offsets[e], offsets[e+1])
// of the sorted rows (forward_prefill.rs page, expert_offsets of
// moe_sort_by_expert).  A launch may also carry the shared expert as one more
// group after the routed ones, holding all N tokens as rows [0, N) of its own
// (run_shared_expert_prefill on the same page: a dense MLP over every token).
// Group e needs ceil(rows_e / BM) row tiles times its column tiles (the shared
// expert's intermediate size may differ from the routed experts', so a gate/up
// launch has two column-tile counts).  The host only knows an upper bound of the
// tile count, so the grid is sized to that bound (a multiple of 8) and every
// block recomputes the exact per-group tile prefix from the device offsets, then
// either takes a tile or leaves.
//
// Block -> tile map: MI355X hands consecutive workgroups to its 8 XCDs round
// robin, and each XCD has its own L2.  Block b runs on XCD b % 8, so it takes
// logical tile (b % 8) * ceil(T/8) + b / 8: each XCD works through one
// contiguous range of logical tiles.  Within a group the logical order is
// (column tile, row tile) with row tiles fastest, so the blocks that share one
// weight slab run together on one XCD and read it from HBM once.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kMaxGroups = 1024;
constexpr int kMaxSchedWaves = 16;  // tile_prefix's s_wsum: one int per wave of the block, at most this many

// The groups of one launch: routed groups [0, nr) read from offsets, then, if xr > 0, one more group
// (index nr) of rows [0, xr): the shared expert.
struct Groups {
  const int32_t* offsets;
  int nr;   // routed groups
  int xr;   // rows of the shared group (0: none)
  int nt;   // column tiles of a routed group
  int xnt;  // column tiles of the shared group
};

// The groups of a grouped GEMM launch whose tiles cover COLS output columns: gate/up (stage 0) has I
// output columns per routed expert and Is for the shared one, down has H for both.
__host__ __device__ inline Groups gemm_groups(const GroupedGemmArgs& g, int stage, int COLS) {
  Groups G;
  G.offsets = g.offsets;
  G.nr = g.shared ? 0 : g.E;
  G.xr = (g.shared || g.with_shared) ? g.N : 0;
  G.nt = (stage == 0 ? g.I : g.H) / COLS;
  G.xnt = (stage == 0 ? g.Is : g.H) / COLS;
  return G;
}

struct TileCoord {
  int expert;   // -1: this block has no tile; the shared group has index Groups::nr
  int m_tile;
  int n_tile;
  int row0;     // first row of the tile (sorted row; a token for the shared group)
  int row_end;  // end of the tile's rows: the segment's end, or the next tile's first row (even split)
  int m_tiles;  // row tiles over all groups (the tiles of one column tile) when every group has the same
                // column-tile count, else -1
};

// rows of group e (0 past the last group)
__device__ __forceinline__ int group_rows(const Groups& G, int e) {
  if (e < G.nr) return G.offsets[e + 1] - G.offsets[e];
  return e == G.nr ? G.xr : 0;
}

// The tile prefix of a launch's groups: s_prefix[e] = tiles (row tiles x column tiles) of the groups
// before e, s_prefix[ngroups] = all tiles, which is returned to every thread.  s_prefix holds at least
// ngroups + 1 ints of LDS (ngroups = G.nr + (G.xr > 0) <= kMaxGroups), s_wsum one int per wave (every
// wave writes its sum, the groups' sums being in the first four); block of 256 to 64 kMaxSchedWaves
// threads, all of which call.
__device__ __forceinline__ int tile_prefix(const Groups& G, int BM, int* s_prefix, int* s_wsum) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int ngroups = G.nr + (G.xr > 0 ? 1 : 0);
  // each thread owns 4 consecutive groups.  Their row counts come from offsets[4 tid .. 4 tid + 4]
  // (clamped to the table), all five loads issued before the first is used: one memory round trip
  // rather than one per group.
  int rows[4];
  if (G.nr > 0) {  // (a launch of the shared expert alone has no offsets table)
    int off[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) off[k] = G.offsets[min(tid * 4 + k, G.nr)];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid * 4 + j;
      rows[j] = e < G.nr ? off[j + 1] - off[j] : (e == G.nr ? G.xr : 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) rows[j] = tid * 4 + j == 0 ? G.xr : 0;
  }
  int cnt[4], local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * 4 + j;
    cnt[j] = e < ngroups ? (rows[j] + BM - 1) / BM * (e < G.nr ? G.nt : G.xnt) : 0;
    local += cnt[j];
  }
  // inclusive scan of `local` across the block
  int incl = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wsum[w];
  int run = before + incl - local;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * 4 + j;
    if (e < ngroups) s_prefix[e] = run;
    run += cnt[j];
  }
  if (tid == 0) s_prefix[ngroups] = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
  __syncthreads();
  return s_prefix[ngroups];
}

// The tile at logical index L of a launch whose tile prefix is s_prefix (T tiles in all; L < T).
// split_align == 0: a segment's tiles start every BM rows, the last one ragged.  split_align > 0 (a
// divisor of BM): the segment is cut into the same number of tiles, of ceil(rows / tiles) rows
// rounded up to split_align, so its tiles carry nearly equal work (130 rows: 96 + 34, not 128 + 2).
__device__ __forceinline__ TileCoord tile_at(const Groups& G, int BM, const int* s_prefix, int T, int L,
                                             int split_align = 0) {
  const int ngroups = G.nr + (G.xr > 0 ? 1 : 0);
  TileCoord tc{-1, 0, 0, 0, 0, G.nt == G.xnt || G.xr == 0 ? T / G.nt : -1};
  // largest e with s_prefix[e] <= L
  int lo = 0, hi = ngroups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (s_prefix[mid] <= L) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  int seg0 = 0, seg_end = G.xr;  // the shared group: rows [0, xr)
  if (e < G.nr) {  // both offsets under one test, so that the two loads share one round trip
    seg0 = G.offsets[e];
    seg_end = G.offsets[e + 1];
  }
  const int mt_e = (seg_end - seg0 + BM - 1) / BM;
  const int rem = L - s_prefix[e];
  tc.expert = e;
  tc.n_tile = rem / mt_e;
  tc.m_tile = rem % mt_e;
  // rows per tile: BM, or the even split (never above BM, and mt_e - 1 tiles of it stay below the
  // segment's rows, so every tile is non-empty)
  int rpt = BM;
  if (split_align > 0 && mt_e > 1) {
    const int even = (seg_end - seg0 + mt_e - 1) / mt_e;
    rpt = (even + split_align - 1) / split_align * split_align;
  }
  tc.row0 = seg0 + tc.m_tile * rpt;
  tc.row_end = min(tc.row0 + rpt, seg_end);
  return tc;
}

// tile_at for a wave-uniform L, with the segment bounds read by scalar loads: a kernel that keeps direct
// global -> LDS loads in flight while it finds its next tile then waits only on those two words, not on
// every vector load issued before them.  The same result as tile_at.
__device__ __forceinline__ TileCoord tile_at_uniform(const Groups& G, int BM, const int* s_prefix, int T, int L,
                                                     int split_align = 0) {
  const int ngroups = G.nr + (G.xr > 0 ? 1 : 0);
  TileCoord tc{-1, 0, 0, 0, 0, G.nt == G.xnt || G.xr == 0 ? T / G.nt : -1};
  int lo = 0, hi = ngroups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (s_prefix[mid] <= L) lo = mid;
    else hi = mid - 1;
  }
  const int e = __builtin_amdgcn_readfirstlane(lo);
  int seg0 = 0, seg_end = G.xr;
  if (e < G.nr) {
    typedef const int __attribute__((address_space(4)))* const_int_ptr;
    const_int_ptr off = (const_int_ptr)(G.offsets);
    seg0 = off[e];
    seg_end = off[e + 1];
  }
  const int mt_e = (seg_end - seg0 + BM - 1) / BM;
  const int rem = L - __builtin_amdgcn_readfirstlane(s_prefix[e]);
  tc.expert = e;
  tc.n_tile = rem / mt_e;
  tc.m_tile = rem % mt_e;
  int rpt = BM;
  if (split_align > 0 && mt_e > 1) {
    const int even = (seg_end - seg0 + mt_e - 1) / mt_e;
    rpt = (even + split_align - 1) / split_align * split_align;
  }
  tc.row0 = seg0 + tc.m_tile * rpt;
  tc.row_end = min(tc.row0 + rpt, seg_end);
  return tc;
}

// Entry e (wave-uniform) of a device table of pointers, by a scalar load (see tile_at_uniform).
template <typename T>
__device__ __forceinline__ T* table_entry_uniform(T* const* table, int e) {
  typedef T* const __attribute__((address_space(4)))* const_table;
  return ((const_table)table)[e];
}

// The tile of block slot `b` (blockIdx.x unless one launch runs several grids of tiles), or expert -1
// when the slot has none: tile_prefix, then the XCD-aware map of slots to logical tiles.  s_prefix must
// hold kMaxGroups + 1 ints in LDS.
__device__ __forceinline__ TileCoord schedule_tile_at(const Groups& G, int BM, int* s_prefix, int* s_wsum, int b,
                                                      int split_align = 0) {
  const int T = tile_prefix(G, BM, s_prefix, s_wsum);
  const int chunk = (T + 7) / 8;
  const int local_idx = b / 8;
  const int L = (b % 8) * chunk + local_idx;
  if (local_idx >= chunk || L >= T) return TileCoord{-1, 0, 0, 0, 0, G.nt == G.xnt || G.xr == 0 ? T / G.nt : -1};
  return tile_at(G, BM, s_prefix, T, L, split_align);
}

__device__ __forceinline__ TileCoord schedule_tile(const Groups& G, int BM, int* s_prefix, int* s_wsum,
                                                   int split_align = 0) {
  return schedule_tile_at(G, BM, s_prefix, s_wsum, blockIdx.x, split_align);
}

// Grid size for a grouped GEMM: an upper bound of the tile count, rounded up to 8.
inline unsigned grouped_grid(int rows_upper, int num_groups, int BM, int NT) {
  long mt = (long)rows_upper / BM + (rows_upper < num_groups ? rows_upper : num_groups) + 1;
  long t = mt * NT;
  t = (t + 7) / 8 * 8;
  return (unsigned)t;
}

// The same bound for a launch's groups (routed rows P = N K at most, plus the shared group's rows).
inline unsigned grouped_grid(const GroupedGemmArgs& g, const Groups& G, int BM) {
  const int rows = (G.nr > 0 ? g.P : 0) + G.xr;
  const int groups = G.nr + (G.xr > 0 ? 1 : 0);
  return grouped_grid(rows, groups, BM, G.nt > G.xnt ? G.nt : G.xnt);
}

}  // namespace moe
