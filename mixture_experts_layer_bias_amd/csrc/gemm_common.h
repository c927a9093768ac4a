// Device-side tile scheduler shared by the grouped expert GEMMs.
//
// The rows of each expert are a contiguous segment [offsets[e], offsets[e+1])
// of the sorted rows (forward_prefill.rs page, expert_offsets of
// moe_sort_by_expert).  Expert e needs ceil(count_e / BM) row tiles times NT
// column tiles.  The host only knows an upper bound of the tile count, so the
// grid is sized to that bound (a multiple of 8) and every block recomputes the
// exact per-expert tile prefix from the device offsets, then either takes a
// tile or leaves.
//
// Block -> tile map: MI355X hands consecutive workgroups to its 8 XCDs round
// robin, and each XCD has its own L2.  Block b runs on XCD b % 8, so it takes
// logical tile (b % 8) * ceil(T/8) + b / 8: each XCD works through one
// contiguous range of logical tiles.  Within an expert the logical order is
// (column tile, row tile) with row tiles fastest, so the blocks that share one
// weight slab run together on one XCD and read it from HBM once.
#pragma once

#include "common.h"

namespace moe {

constexpr int kMaxGroups = 1024;

struct TileCoord {
  int expert;   // -1: this block has no tile
  int m_tile;
  int n_tile;
  int row0;     // first sorted row of the tile
  int row_end;  // end of the tile's rows: the segment's end, or the next tile's first row (even split)
  int m_tiles;  // row tiles over all groups (the tiles of one column tile)
};

// s_prefix must hold kMaxGroups + 1 ints in LDS.  Block of at least 256 threads.  `b` is the
// block's tile slot (blockIdx.x unless one launch runs several grids of tiles).
// split_align == 0: a segment's tiles start every BM rows, the last one ragged.  split_align > 0 (a
// divisor of BM): the segment is cut into the same number of tiles, of ceil(rows / tiles) rows
// rounded up to split_align, so its tiles carry nearly equal work (130 rows: 96 + 34, not 128 + 2).
__device__ __forceinline__ TileCoord schedule_tile_at(const int32_t* __restrict__ offsets, int num_groups,
                                                      int shared_rows, int BM, int NT, int* s_prefix, int* s_wsum,
                                                      int b, int split_align = 0) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  // each thread owns 4 consecutive groups
  int cnt[4], local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * 4 + j;
    int c = 0;
    if (e < num_groups) c = shared_rows >= 0 ? shared_rows : (offsets[e + 1] - offsets[e]);
    cnt[j] = (c + BM - 1) / BM;
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
    if (e < num_groups) s_prefix[e] = run;
    run += cnt[j];
  }
  if (tid == 0) s_prefix[num_groups] = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
  __syncthreads();

  TileCoord tc{-1, 0, 0, 0, 0, s_prefix[num_groups]};
  const int T = s_prefix[num_groups] * NT;
  const int chunk = (T + 7) / 8;
  const int local_idx = b / 8;
  if (local_idx >= chunk) return tc;
  const int L = (b % 8) * chunk + local_idx;
  if (L >= T) return tc;
  // largest e with s_prefix[e] * NT <= L
  int lo = 0, hi = num_groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (s_prefix[mid] * NT <= L) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int mt_e = s_prefix[e + 1] - s_prefix[e];
  const int rem = L - s_prefix[e] * NT;
  tc.expert = e;
  tc.n_tile = rem / mt_e;
  tc.m_tile = rem % mt_e;
  const int seg0 = shared_rows >= 0 ? 0 : offsets[e];
  const int seg_end = shared_rows >= 0 ? shared_rows : offsets[e + 1];
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

__device__ __forceinline__ TileCoord schedule_tile(const int32_t* __restrict__ offsets, int num_groups, int shared_rows,
                                                   int BM, int NT, int* s_prefix, int* s_wsum, int split_align = 0) {
  return schedule_tile_at(offsets, num_groups, shared_rows, BM, NT, s_prefix, s_wsum, blockIdx.x, split_align);
}

// Grid size for a grouped GEMM: an upper bound of the tile count, rounded up to 8.
inline unsigned grouped_grid(int rows_upper, int num_groups, int BM, int NT) {
  long mt = (long)rows_upper / BM + (rows_upper < num_groups ? rows_upper : num_groups) + 1;
  long t = mt * NT;
  t = (t + 7) / 8 * 8;
  return (unsigned)t;
}

}  // namespace moe
