// Stable counting sort of the expanded (token, slot) rows by expert, for gfx950.
// forward_prefill.rs page, moe_sort_by_expert: sorted_token_ids, expert_offsets
// and token_to_perm (here sorted_ids, offsets and inv_perm).
//
// Three passes over chunks of kChunk expanded rows (one wave per 64 rows):
//   count   - per-chunk histograms in LDS                        (one block per chunk)
//   scan    - per bucket, the exclusive prefix of its counts over the chunks and the
//             bucket total (one wave per bucket, a DPP scan across the chunks)
//   scatter - every block turns the bucket totals into bucket offsets (a block scan;
//             block 0 also writes counts and offsets), then each wave ranks its 64 rows:
//             the lanes holding the same id are found with one ballot per id bit, so a
//             row's rank among equal ids below it is a popcount, and equal ids keep
//             ascending expanded index (stable).
// When every scatter block can read all the chunks' counts in one batch of loads
// (C x R / 4 <= 256 x 32), the scan pass is left out: each scatter block adds up
// the counts of the chunks before its own and of all chunks itself (two launches).
// Every step is integer arithmetic with a fixed order, so the result is the same
// on every run.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kChunk = 256;        // expanded rows per chunk (4 waves x 64)
constexpr int kMaxBuckets = 1024;  // router width limit
constexpr int kIdBits = 10;        // ids < kMaxBuckets

int permute_chunks(int P) { return (P + kChunk - 1) / kChunk; }

// hist row c (stride rs >= R ints) <- the counts of chunk c
__global__ __launch_bounds__(256) void k_perm_count(const int32_t* __restrict__ ids, int P, int R, int rs,
                                                    int32_t* __restrict__ hist) {
  __shared__ int h[kMaxBuckets];
  for (int r = threadIdx.x; r < R; r += 256) h[r] = 0;
  __syncthreads();
  const int idx = blockIdx.x * kChunk + threadIdx.x;
  if (idx < P) {
    const int id = ids[idx];
    if ((unsigned)id < (unsigned)R) atomicAdd(&h[id], 1);  // an id outside [0, R) is dropped, never written
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += 256) hist[(size_t)blockIdx.x * rs + r] = h[r];
}

// inclusive wave scan (lane order)
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int x = __shfl_up(v, o, kWave);
    if (lane >= o) v += x;
  }
  return v;
}

// hist[c][r] <- rows of bucket r in chunks before c; totals[r] <- rows of bucket r
__global__ __launch_bounds__(256) void k_perm_scan(int32_t* __restrict__ hist, int C, int R,
                                                   int32_t* __restrict__ totals) {
  const int lane = threadIdx.x % kWave;
  const int r = blockIdx.x * 4 + threadIdx.x / kWave;
  if (r >= R) return;  // the whole wave leaves
  int carry = 0;
  for (int c0 = 0; c0 < C; c0 += 4 * kWave) {  // four batches of 64 chunks in flight
    int v[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int c = c0 + b * kWave + lane;
      v[b] = c < C ? hist[(size_t)c * R + r] : 0;
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int c = c0 + b * kWave + lane;
      const int incl = wave_incl_scan(v[b]);
      if (c < C) hist[(size_t)c * R + r] = carry + incl - v[b];
      carry += __shfl(incl, kWave - 1, kWave);
    }
  }
  if (lane == 0) totals[r] = carry;
}

// The scatter of chunk blockIdx.x once s_base[r] holds, for each bucket, the sorted position of the
// chunk's first row of that bucket.  s_wcnt is zero on entry.
__device__ __forceinline__ void scatter_chunk(const int32_t* __restrict__ ids, int P, int R, int* s_base,
                                              int (*s_wcnt)[kMaxBuckets], int32_t* __restrict__ sorted_ids,
                                              int32_t* __restrict__ inv_perm) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  // this wave's row and its id
  const int idx = blockIdx.x * kChunk + tid;
  const int id = idx < P ? ids[idx] : -1;
  const int v = (unsigned)id < (unsigned)R ? id : -1;
  if (v >= 0) atomicAdd(&s_wcnt[wave][v], 1);
  __syncthreads();
  // per-wave cursors: the chunk cursor plus the rows of the same bucket in earlier waves
  for (int r = tid; r < R; r += 256) {
    int cur = s_base[r];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = s_wcnt[w][r];
      s_wcnt[w][r] = cur;
      cur += c;
    }
  }
  __syncthreads();
  // lanes holding the same id: agree on every id bit (invalid rows have no valid id)
  uint64_t same = __ballot(v >= 0);
#pragma unroll
  for (int b = 0; b < kIdBits; ++b) {
    const uint64_t ones = __ballot(v >= 0 && ((v >> b) & 1));
    same &= ((v >> b) & 1) ? ones : ~ones;
  }
  if (v >= 0) {
    const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int pos = s_wcnt[wave][v] + __popcll(same & lt_mask);
    sorted_ids[pos] = idx;
    inv_perm[idx] = pos;
  }
}

// Bucket offsets from the bucket totals tot(r) (a block scan; each thread owns 4 consecutive buckets):
// s_base[r] <- offset of bucket r + pre(r); block 0 also writes counts and offsets.
template <typename Tot, typename Pre>
__device__ __forceinline__ void bucket_bases(int R, Tot tot, Pre pre, int* s_base, int* s_wsum,
                                             int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  int t4[4], local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = tid * 4 + j;
    t4[j] = r < R ? tot(r) : 0;
    local += t4[j];
  }
  const int incl = wave_incl_scan(local);
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wave; ++w) run += s_wsum[w];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = tid * 4 + j;
    if (r < R) {
      s_base[r] = run + pre(r);
      if (blockIdx.x == 0) {
        counts[r] = t4[j];
        offsets[r] = run;
        if (r == R - 1) offsets[R] = run + t4[j];  // rows with a valid id (P when every id is in range)
      }
    }
    run += t4[j];
  }
}

__global__ __launch_bounds__(256) void k_perm_scatter(const int32_t* __restrict__ ids, int P, int R,
                                                      const int32_t* __restrict__ chunk_prefix,
                                                      const int32_t* __restrict__ totals,
                                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted_ids,
                                                      int32_t* __restrict__ inv_perm, int32_t* __restrict__ clear8) {
  __shared__ int s_base[kMaxBuckets];  // bucket offsets, then this chunk's cursors
  __shared__ int s_wcnt[4][kMaxBuckets];  // rows per bucket in each wave, then per-wave cursors
  __shared__ int s_wsum[4];
  if (clear8 != nullptr && blockIdx.x == 0 && threadIdx.x < 8) clear8[threadIdx.x] = 0;
  for (int i = threadIdx.x; i < 4 * kMaxBuckets; i += 256) (&s_wcnt[0][0])[i] = 0;
  bucket_bases(
      R, [&](int r) { return totals[r]; }, [&](int r) { return chunk_prefix[(size_t)blockIdx.x * R + r]; }, s_base,
      s_wsum, counts, offsets);
  __syncthreads();
  scatter_chunk(ids, P, R, s_base, s_wcnt, sorted_ids, inv_perm);
}

// The scatter of the two-launch sort: hist holds the C chunks' raw counts, rows of rs = 4 R4 ints
// (R4 = ceil(R / 4)).  Thread (q, g) = (tid % R4, tid / R4), for g < G = 256 / R4, adds buckets
// 4q .. 4q + 3 of chunks g, g + G, ... (at most kDirectLoads of them, loaded as one batch), into the
// chunks before this one and into all chunks; the G partial sums per bucket are added in g order.
constexpr int kDirectLoads = 32;

__global__ __launch_bounds__(256) void k_perm_scatter_hist(const int32_t* __restrict__ ids, int P, int R, int C,
                                                           const int32_t* __restrict__ hist,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_ids,
                                                           int32_t* __restrict__ inv_perm,
                                                           int32_t* __restrict__ clear8) {
  __shared__ int s_base[kMaxBuckets];
  __shared__ int s_wcnt[4][kMaxBuckets];  // the partial sums (before and all), then as k_perm_scatter
  __shared__ int s_wsum[4];
  const int tid = threadIdx.x;
  if (clear8 != nullptr && blockIdx.x == 0 && tid < 8) clear8[tid] = 0;
  const int R4 = (R + 3) / 4, rs = 4 * R4, G = 256 / R4;
  const int q = tid % R4, g = tid / R4, c_self = blockIdx.x;
  int* s_pre = &s_wcnt[0][0];  // [G][rs], G rs <= 1024
  int* s_all = &s_wcnt[2][0];
  if (g < G) {
    u32x4 v[kDirectLoads];
#pragma unroll
    for (int j = 0; j < kDirectLoads; ++j) {
      const int c = min(g + G * j, C - 1);  // past the last chunk: reload it, add nothing
      v[j] = ldg16(hist + (size_t)c * rs + 4 * q);
    }
    int pre[4] = {0, 0, 0, 0}, all[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kDirectLoads; ++j) {
      const int c = g + G * j;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int x = (c < C && 4 * q + e < R) ? (int)v[j][e] : 0;  // a row's padding is never written
        all[e] += x;
        pre[e] += c < c_self ? x : 0;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s_pre[g * rs + 4 * q + e] = pre[e];
      s_all[g * rs + 4 * q + e] = all[e];
    }
  }
  __syncthreads();
  auto sum_over = [&](const int* a, int r) {
    int t = 0;
    for (int gg = 0; gg < G; ++gg) t += a[gg * rs + r];
    return t;
  };
  bucket_bases(
      R, [&](int r) { return sum_over(s_all, r); }, [&](int r) { return sum_over(s_pre, r); }, s_base, s_wsum,
      counts, offsets);
  __syncthreads();
  for (int i = tid; i < 4 * kMaxBuckets; i += 256) (&s_wcnt[0][0])[i] = 0;
  __syncthreads();
  scatter_chunk(ids, P, R, s_base, s_wcnt, sorted_ids, inv_perm);
}

bool permute_direct(int P, int R) {
  const long C = permute_chunks(P);
  return C > 0 && C * ((R + 3) / 4) <= 256L * kDirectLoads;
}

hipError_t launch_permute(const int32_t* ids, int P, int R, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                          int32_t* inv_perm, int32_t* hist, int32_t* clear8, hipStream_t s) {
  const int C = permute_chunks(P);
  if (permute_direct(P, R)) {
    k_perm_count<<<C, 256, 0, s>>>(ids, P, R, 4 * ((R + 3) / 4), hist);
    k_perm_scatter_hist<<<C, 256, 0, s>>>(ids, P, R, C, hist, counts, offsets, sorted_ids, inv_perm, clear8);
    return hipGetLastError();
  }
  int32_t* totals = hist + (size_t)C * R;  // R more ints after the chunk histograms
  if (C > 0) k_perm_count<<<C, 256, 0, s>>>(ids, P, R, R, hist);
  k_perm_scan<<<(R + 3) / 4, 256, 0, s>>>(hist, C, R, totals);
  k_perm_scatter<<<C > 0 ? C : 1, 256, 0, s>>>(ids, P, R, hist, totals, counts, offsets, sorted_ids, inv_perm,
                                                clear8);
  return hipGetLastError();
}

}  // namespace moe
