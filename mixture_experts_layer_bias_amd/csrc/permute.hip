// Stable counting sort of the expanded (token, slot) rows by expert, for gfx950.
// forward_prefill.rs page, moe_sort_by_expert: sorted_token_ids, expert_offsets
// and token_to_perm (here sorted_ids, offsets and inv_perm).
//
// Three passes over chunks of kChunk expanded rows:
//   count   - per-chunk histograms in LDS                    (one block per chunk)
//   scan    - per-bucket exclusive prefix over chunks, then over buckets -> counts,
//             offsets, and each chunk's starting cursor per bucket (one block)
//   scatter - each wave ranks its 256 rows in order with ballots, so equal ids keep
//             ascending expanded index (stable), and writes both permutations.
// Every step is integer arithmetic with a fixed order, so the result is the same
// on every run.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kChunk = 1024;     // expanded rows per chunk (4 waves x 256)
constexpr int kMaxBuckets = 1024;  // router width limit

int permute_chunks(int P) { return (P + kChunk - 1) / kChunk; }

__global__ __launch_bounds__(256) void k_perm_count(const int32_t* __restrict__ ids, int P, int R,
                                                    int32_t* __restrict__ hist) {
  __shared__ int h[kMaxBuckets];
  for (int r = threadIdx.x; r < R; r += 256) h[r] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
#pragma unroll
  for (int i = 0; i < kChunk / 256; ++i) {
    int idx = base + i * 256 + threadIdx.x;
    if (idx < P) {
      const int id = ids[idx];
      if ((unsigned)id < (unsigned)R) atomicAdd(&h[id], 1);  // an id outside [0, R) is dropped, never written
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += 256) hist[(size_t)blockIdx.x * R + r] = h[r];
}

__global__ __launch_bounds__(1024) void k_perm_scan(int32_t* __restrict__ hist, int C, int R,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int s[kMaxBuckets];
  const int r = threadIdx.x;
  int total = 0;
  if (r < R)
    for (int c = 0; c < C; ++c) {
      int v = hist[(size_t)c * R + r];
      hist[(size_t)c * R + r] = total;  // rows of bucket r in chunks before c
      total += v;
    }
  s[r] = r < R ? total : 0;
  __syncthreads();
  for (int off = 1; off < kMaxBuckets; off <<= 1) {
    int v = r >= off ? s[r - off] : 0;
    __syncthreads();
    s[r] += v;
    __syncthreads();
  }
  if (r < R) {
    int excl = s[r] - total;
    counts[r] = total;
    offsets[r] = excl;
    for (int c = 0; c < C; ++c) hist[(size_t)c * R + r] += excl;
  }
  if (r == R - 1) offsets[R] = s[r];  // rows with a valid id (P when every id is in range)
}

__global__ __launch_bounds__(256) void k_perm_scatter(const int32_t* __restrict__ ids, int P, int R,
                                                      const int32_t* __restrict__ chunk_base,
                                                      int32_t* __restrict__ sorted_ids,
                                                      int32_t* __restrict__ inv_perm) {
  __shared__ int cur[4][kMaxBuckets];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  for (int i = threadIdx.x; i < 4 * kMaxBuckets; i += 256) (&cur[0][0])[i] = 0;
  __syncthreads();
  const int wbase = blockIdx.x * kChunk + wave * 256;
  int my_id[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int idx = wbase + i * 64 + lane;
    const int id = idx < P ? ids[idx] : -1;
    my_id[i] = (unsigned)id < (unsigned)R ? id : -1;
    if (my_id[i] >= 0) atomicAdd(&cur[wave][my_id[i]], 1);
  }
  __syncthreads();
  // per-wave starting cursors: chunk base + rows of the same bucket in earlier waves
  for (int r = threadIdx.x; r < R; r += 256) {
    int run = chunk_base[(size_t)blockIdx.x * R + r];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      int c = cur[w][r];
      cur[w][r] = run;
      run += c;
    }
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = wbase + i * 64 + lane;
    const int v = my_id[i];
    uint64_t pending = __ballot(v >= 0);
    while (pending) {  // one pass per distinct id in this group of 64 rows (wave-uniform)
      const int leader = __ffsll((unsigned long long)pending) - 1;
      const int lv = __builtin_amdgcn_readlane(v, leader);
      const uint64_t same = __ballot(v == lv);
      if (v == lv) {
        const int pos = cur[wave][lv] + __popcll(same & lt_mask);
        sorted_ids[pos] = idx;
        inv_perm[idx] = pos;
      }
      __builtin_amdgcn_wave_barrier();
      if (lane == leader) cur[wave][lv] += __popcll(same);
      __builtin_amdgcn_wave_barrier();
      pending &= ~same;
    }
  }
}

hipError_t launch_permute(const int32_t* ids, int P, int R, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                          int32_t* inv_perm, int32_t* hist, hipStream_t s) {
  const int C = permute_chunks(P);
  if (C > 0) {
    k_perm_count<<<C, 256, 0, s>>>(ids, P, R, hist);
  }
  k_perm_scan<<<1, 1024, 0, s>>>(hist, C, R, counts, offsets);
  if (C > 0) {
    k_perm_scatter<<<C, 256, 0, s>>>(ids, P, R, hist, sorted_ids, inv_perm);
  }
  return hipGetLastError();
}

}  // namespace moe
