// Router gate GEMM and top-K scoring for gfx950.
//
// Gate GEMM: forward_prefill.rs page (MoeLayer::forward_prefill, gate GEMM
// step) and forward_batched.rs page (the router width counts the
// zero-computation experts).  Scoring and selection: forward.rs page,
// MoeLayer::forward top-K arms (softmax; sigmoid + correction bias for
// selection, unbiased weights renormalised then scaled; softmax + correction
// bias with the zero-expert fold; the DeepSeek-V4 sqrtsoftplus + correction
// bias arm, weighted like the sigmoid one).
#include "common.h"
#include "dma.h"
#include "kernels.h"

namespace moe {

// logits[N, R] = x[N, H] . router_w[R, H]^T on v_mfma_f32_16x16x32_bf16.
// A block of 4 waves computes a 32-token x 64-column tile over one slice of H
// (split-K: blockIdx.z selects the slice; the host picks the number of slices
// so that small batches still spread over the chip).  A and B are staged
// through LDS 128 columns of H at a time, with the next slab's global loads in
// flight during the MFMAs.  Wave w owns columns [16w, 16w+16) and both 16-row
// halves.  Each slice writes its own partial [N, R] plane; the top-K kernel
// adds the planes in slice order, so the sum order is fixed.
constexpr int RT_BM = 32, RT_BN = 64, RT_BK = 128, RT_LDS = RT_BK + 8;  // bf16 elements per LDS row

__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ wr, float* __restrict__ part,
                                                       int N, int H, int R, int kslice) {
  __shared__ __align__(16) uint16_t a_lds[RT_BM * RT_LDS];
  __shared__ __align__(16) uint16_t b_lds[RT_BN * RT_LDS];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int m0 = blockIdx.x * RT_BM, n0 = blockIdx.y * RT_BN;
  const int k_begin = blockIdx.z * kslice;
  // staging: row = tid / 16 (+16 i), 16-byte chunk = tid % 16
  const int lrow = tid >> 4, lcol = (tid & 15) * 8;
  const uint16_t* ap[2];
  const uint16_t* bp[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int row = m0 + lrow + 16 * i;
    row = row < N ? row : N - 1;  // clamp: extra rows are computed, never stored
    ap[i] = x + (size_t)row * H + k_begin + lcol;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int col = n0 + lrow + 16 * i;
    col = col < R ? col : R - 1;
    bp[i] = wr + (size_t)col * H + k_begin + lcol;
  }
  u32x4 ra[2], rb[4];
  auto load = [&](int k) {
#pragma unroll
    for (int i = 0; i < 2; ++i) ra[i] = ldg16(ap[i] + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = ldg16(bp[i] + k);
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) st16(a_lds + (lrow + 16 * i) * RT_LDS + lcol, ra[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) st16(b_lds + (lrow + 16 * i) * RT_LDS + lcol, rb[i]);
  };
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const int frow = lane & 15, fk = (lane >> 4) * 8;
  load(0);
  store();
  __syncthreads();
  const int nk = kslice / RT_BK;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load((kt + 1) * RT_BK);
#pragma unroll
    for (int kk = 0; kk < RT_BK; kk += 32) {
      const u32x4 b = ld16(b_lds + (wave * 16 + frow) * RT_LDS + kk + fk);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const u32x4 a = ld16(a_lds + (mi * 16 + frow) * RT_LDS + kk + fk);
        acc[mi] = mfma_16x16x32_bf16(a, b, acc[mi]);
      }
    }
    __syncthreads();
    if (kt + 1 < nk) {
      store();
      __syncthreads();
    }
  }
  // D layout of the 16x16 MFMA: lane l, item r -> row 4*(l/16) + r, column l%16
  float* out = part + (size_t)blockIdx.z * N * R;
  const int col = n0 + wave * 16 + (lane & 15);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + mi * 16 + (lane >> 4) * 4 + r;
      if (row < N && col < R) out[(size_t)row * R + col] = acc[mi][r];
    }
}

// Router logits for a handful of tokens (N <= RG_MAXN): one wave per router
// column.  Lane l holds 16-byte chunks l, l + 64, ... of the column's weight
// row and of each token's row; each lane adds its products in chunk order and
// the wave adds the 64 lane sums on DPP, so the sum order is fixed.  The
// logits come out whole (no split planes), and every load of a lane is issued
// before its first multiply.
constexpr int RG_MAXN = 8;

__device__ __forceinline__ void bf16x8_to_f32(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

// The calling wave's router column r against the N tokens: acc[t] gets this lane's partial sum of
// token t (wave_sum of it is the logit).
template <int NT, int G>  // NT >= N tokens, G chunks per lane in flight
__device__ __forceinline__ void gemv_column(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int N,
                                            int H, int r, float* acc) {
  const int lane = threadIdx.x % kWave;
  const int nch = H / 8;
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
  for (int c0 = lane; c0 < nch; c0 += G * kWave) {
    u32x4 wv[G], xv[G][NT];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int c = c0 + g * kWave;
      wv[g] = c < nch ? ldg16(wr + (size_t)r * H + c * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < NT; ++t)
        xv[g][t] = (c < nch && t < N) ? ldg16(x + (size_t)t * H + c * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float wf[8];
      bf16x8_to_f32(wv[g], wf);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float xf[8];
        bf16x8_to_f32(xv[g][t], xf);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[t] = fmaf(wf[e], xf[e], acc[t]);
      }
    }
  }
}

template <int NT, int G>
__global__ __launch_bounds__(256) void k_router_gemv(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                     float* __restrict__ logits, int N, int H, int R) {
  const int lane = threadIdx.x % kWave;
  const int r = blockIdx.x * 4 + threadIdx.x / kWave;
  if (r >= R) return;  // the whole wave leaves
  float acc[NT];
  gemv_column<NT, G>(x, wr, N, H, r, acc);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < N) {  // uniform
      const float s = wave_sum(acc[t]);
      if (lane == 0) logits[(size_t)t * R + r] = s;
    }
  }
}

// One wave per token: scores in fp32, then K rounds of a wave-wide arg-max:
// the largest order-preserving key of the selection scores (a DPP max), then a
// ballot for the lowest column holding it, so ties go to the lower column and
// slots come out in descending order.  MAXJ = ceil(R/64) scores per lane.
__device__ __forceinline__ uint32_t order_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#define MOE_STEP(C, M) v = max(v, dpp_u32<C, M>(0u, v))
  MOE_STEP(kDppRowShr1, 0xF);
  MOE_STEP(kDppRowShr2, 0xF);
  MOE_STEP(kDppRowShr4, 0xF);
  MOE_STEP(kDppRowShr8, 0xF);
  MOE_STEP(kDppRowBcast15, 0xA);
  MOE_STEP(kDppRowBcast31, 0xC);
#undef MOE_STEP
  return __builtin_amdgcn_readlane(v, 63);
}

// Scores and top-K of token t for the calling wave.  p_w is this wave's LDS row
// of MAXJ*64 floats.  Returns the wave's slot id (lane k holds slot k's column;
// lanes >= K hold 0) after writing ids / w / zero_w for the token.  TAGGED: `part` holds, for every
// (token, column), a 64-bit word (seq << 32 | logit bits) that other blocks of this launch store at
// device scope; the wave reads them at device scope until every word carries `seq` (at most
// kRouteSpinLimit rounds; past it *expired is set and the values are undefined), writes the logits out and
// puts the words back to zero, so that the next launch, which may repeat `seq` (a graph replay), waits
// for its own.
constexpr int kRouteSpinLimit = 1 << 20;

template <int MAXJ, bool TAGGED = false>
__device__ __forceinline__ int topk_token(const float* __restrict__ part, int nslices, float* __restrict__ logits,
                                          const float* __restrict__ bias, int32_t* __restrict__ ids,
                                          float* __restrict__ w, float* __restrict__ zero_w, float* p_w, int t, int N,
                                          int R, int E, int K, int scoring, int renorm, float scale,
                                          uint32_t seq = 0, int* expired = nullptr) {
  const int lane = threadIdx.x % kWave;
  // logits of this token: the split-K partial planes added in slice order
  float v[MAXJ];
  if (TAGGED) {
    unsigned long long* tw =
        reinterpret_cast<unsigned long long*>(const_cast<float*>(part)) + (size_t)t * R;
    unsigned long long word[MAXJ];
    bool ready = false;
    for (int it = 0; it < kRouteSpinLimit && !ready; ++it) {
      ready = true;
#pragma unroll
      for (int j = 0; j < MAXJ; ++j) {
        const int r = lane + 64 * j;
        if (r < R && (it == 0 || (uint32_t)(word[j] >> 32) != seq))
          word[j] = __hip_atomic_load(tw + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int j = 0; j < MAXJ; ++j)
        if (lane + 64 * j < R && (uint32_t)(word[j] >> 32) != seq) ready = false;
      ready = __all(ready);
      if (!ready) __builtin_amdgcn_s_sleep(1);
    }
    if (!ready && lane == 0) *expired = 1;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int r = lane + 64 * j;
      if (r < R) {
        v[j] = __uint_as_float((uint32_t)word[j]);
        logits[(size_t)t * R + r] = v[j];
        __hip_atomic_store(tw + r, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        v[j] = -INFINITY;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    if (TAGGED) break;
    const int r = lane + 64 * j;
    if (r < R && nslices == 1) {  // whole logits (the GEMV router): one load
      v[j] = part[(size_t)t * R + r];
    } else if (r < R) {
      // all planes are loaded before the (in-order) additions, so the loads overlap
      float pl[16];
#pragma unroll
      for (int z = 0; z < 16; ++z) pl[z] = z < nslices ? part[((size_t)z * N + t) * R + r] : 0.f;
      float acc = pl[0];
#pragma unroll
      for (int z = 1; z < 16; ++z)
        if (z < nslices) acc += pl[z];
      v[j] = acc;
      logits[(size_t)t * R + r] = acc;
    } else {
      v[j] = -INFINITY;
    }
  }
  float p[MAXJ];
  if (scoring == 0) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) m = fmaxf(m, v[j]);
    m = wave_max(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      p[j] = (lane + 64 * j) < R ? expf(v[j] - m) : 0.f;
      s += p[j];
    }
    s = wave_sum(s);
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) p[j] = p[j] / s;
  } else if (scoring == 1) {
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      int r = lane + 64 * j;
      p[j] = r < R ? 1.0f / (1.0f + expf(-v[j])) : 0.f;
    }
  } else {  // sqrt(softplus(z)), softplus(z) = ln(1 + e^z) = max(z, 0) + ln(1 + e^-|z|)
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      int r = lane + 64 * j;
      p[j] = r < R ? sqrtf(fmaxf(v[j], 0.f) + log1pf(expf(-fabsf(v[j])))) : 0.f;
    }
  }
  float sel[MAXJ];
  uint32_t avail = 0;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    int r = lane + 64 * j;
    if (r < R) {
      p_w[r] = p[j];
      sel[j] = bias ? p[j] + bias[r] : p[j];
      avail |= 1u << j;
    } else {
      sel[j] = 0.f;
    }
  }
  // K rounds: the largest key left, then the lowest column holding it (ties go to the
  // lower column; the key order is the score order, so slots come out descending)
  uint32_t key[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) key[j] = order_bits(sel[j]);
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    uint32_t best = 0;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j)
      if ((avail >> j) & 1u) best = key[j] > best ? key[j] : best;
    best = wave_max_u32(best);
    // the lowest column holding it: slices from the top, so the lowest slice with a hit is the
    // last to set r_star (selects, no branches)
    int r_star = 0;
#pragma unroll
    for (int j = MAXJ - 1; j >= 0; --j) {
      const uint64_t hit = __ballot(((avail >> j) & 1u) && key[j] == best);
      r_star = hit ? 64 * j + (int)__builtin_ctzll(hit) : r_star;
    }
    if (lane == (r_star & 63)) avail &= ~(1u << (r_star >> 6));
    if (lane == k) my_id = r_star;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float my_p = lane < K ? p_w[my_id] : 0.f;
  float wk = my_p;
  if (renorm) {
    float tot = wave_sum(my_p);
    wk = my_p / tot;
  }
  wk *= scale;
  float zsum = wave_sum((lane < K && my_id >= E) ? wk : 0.f);
  if (lane < K) {
    ids[(size_t)t * K + lane] = my_id;
    w[(size_t)t * K + lane] = wk;
  }
  if (lane == 0 && zero_w) zero_w[t] = zsum;
  return my_id;
}

template <int MAXJ>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ part, int nslices,
                                              float* __restrict__ logits, const float* __restrict__ bias,
                                              int32_t* __restrict__ ids, float* __restrict__ w,
                                              float* __restrict__ zero_w, int N, int R, int E, int K, int scoring,
                                              int renorm, float scale) {
  __shared__ float p_lds[4][MAXJ * 64];
  const int wave = threadIdx.x / kWave;
  const int t = blockIdx.x * 4 + wave;
  if (t >= N) return;  // the whole wave leaves; no block barrier below
  topk_token<MAXJ>(part, nslices, logits, bias, ids, w, zero_w, p_lds[wave], t, N, R, E, K, scoring, renorm, scale);
}

// The stable counting sort of up to 64 expanded rows, by one wave: s_ids (LDS) holds the P <= 64 row
// ids, s_off (LDS) at least R ints, zero on entry.  Lane p holds row p's id v; one ballot per id bit,
// from the top, splits the rows into those with a smaller id (lt) and those with the same id (eq), so
// row p lands at |lt| + |{q in eq : q < p}|.
__device__ __forceinline__ void sort_rows_ballot(const int* s_ids, int* s_off, int P, int R, int32_t* counts,
                                                 int32_t* offsets, int32_t* sorted_ids, int32_t* inv_perm) {
  const int lane = threadIdx.x % kWave;
  const bool valid = lane < P;
  const int v = valid ? s_ids[lane] : 0;
  uint64_t eq = __ballot(valid), lt = 0;
  for (int b = 31 - __builtin_clz((unsigned)R); b >= 0; --b) {  // ids < R fit in these bits
    const bool bit = (v >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    if (bit) {
      lt |= eq & ~ones;
      eq &= ones;
    } else {
      eq &= ~ones;
    }
  }
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));  // lanes before this one
  const int rank = __popcll(eq & below);
  if (valid) {
    const int pos = __popcll(lt) + rank;
    sorted_ids[pos] = lane;
    inv_perm[lane] = pos;
    if (rank == 0) s_off[v] = __popcll(eq);  // the expert's first row writes its count
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // exclusive scan of the R counts: lane l owns buckets [l C, l C + C)
  const int C = (R + kWave - 1) / kWave;
  int sum = 0;
  for (int c = 0; c < C; ++c) {
    const int r = lane * C + c;
    if (r < R) sum += s_off[r];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int xo = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += xo;
  }
  int run = incl - sum;
  for (int c = 0; c < C; ++c) {
    const int r = lane * C + c;
    if (r < R) {
      const int cnt = s_off[r];
      counts[r] = cnt;
      offsets[r] = run;
      run += cnt;
    }
  }
  if (lane == kWave - 1) offsets[R] = incl;  // = P
}

// Small batches (N <= 64, N*K <= 1024): top-K of every token and the stable
// counting sort by expert in ONE block of 16 waves, so a decode step spends one
// launch on both (same results as k_topk followed by the three sort passes).
// Expanded row i of expert e lands at offsets[e] + (the number of rows j < i of
// expert e): up to 64 rows, one wave finds it from ballots; otherwise every row
// counts it from LDS broadcast reads of the ids.
template <int MAXJ>
__global__ __launch_bounds__(1024) void k_topk_sort_small(const float* __restrict__ part, int nslices,
                                                         float* __restrict__ logits, const float* __restrict__ bias,
                                                         int32_t* __restrict__ ids, float* __restrict__ w,
                                                         float* __restrict__ zero_w, int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted_ids,
                                                         int32_t* __restrict__ inv_perm, int32_t* __restrict__ done,
                                                         int done_len, int N, int R, int E, int K, int scoring,
                                                         int renorm, float scale) {
  __shared__ float p_lds[16][MAXJ * 64];
  __shared__ __align__(16) int s_ids[1024];
  __shared__ int s_off[1024];  // bucket counts, then bucket offsets
  __shared__ int s_wsum[16];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int P = N * K;
  if (tid < R) s_off[tid] = 0;
  if (done)
    for (int i = tid; i < done_len; i += 1024) done[i] = 0;
  for (int t = wave; t < N; t += 16) {
    const int my_id = topk_token<MAXJ>(part, nslices, logits, bias, ids, w, zero_w, p_lds[wave], t, N, R, E, K,
                                       scoring, renorm, scale);
    if (lane < K) s_ids[t * K + lane] = my_id;
  }
  __syncthreads();
  if (P <= kWave) {  // up to 64 rows (decode): wave 0 sorts them with ballots
    if (wave == 0) sort_rows_ballot(s_ids, s_off, P, R, counts, offsets, sorted_ids, inv_perm);
    return;
  }
  // one expanded row per thread, in order
  const int v = tid < P ? s_ids[tid] : -1;
  if (v >= 0) atomicAdd(&s_off[v], 1);
  __syncthreads();
  // exclusive scan over the buckets (thread b owns bucket b): a wave scan, then the
  // wave totals added in order
  const int total = tid < R ? s_off[tid] : 0;
  int incl = total;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int xo = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += xo;
  }
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int ww = 0; ww < wave; ++ww) before += s_wsum[ww];
  incl += before;
  if (tid < R) {
    counts[tid] = total;
    offsets[tid] = incl - total;
    s_off[tid] = incl - total;
    if (tid == R - 1) offsets[R] = incl;
  }
  __syncthreads();
  if (v >= 0) {
    int rank = 0, j = 0;
    for (; j + 4 <= tid; j += 4) {
      const int4 q = *reinterpret_cast<const int4*>(&s_ids[j]);
      rank += (q.x == v) + (q.y == v) + (q.z == v) + (q.w == v);
    }
    for (; j < tid; ++j) rank += s_ids[j] == v;
    const int pos = s_off[v] + rank;
    sorted_ids[pos] = tid;
    inv_perm[tid] = pos;
  }
}

// The decode prelude in one launch (N <= 8 tokens, N K <= 64 rows, R <= 1024): router GEMV, top-K and
// the sort, with the same results as k_router_gemv followed by k_topk_sort_small.  Every block of 8
// waves computes 8 router columns (one per wave) and stores each logit at device scope as one 64-bit
// word tagged with `seq` (a nonzero value of this launch that differs from the last launch's on the same
// words).  Block 0 then runs the top-K of each token (one wave per token), reading its logits at device
// scope until every word carries seq (a bounded wait), puts the words back to 0, and runs the ballot
// sort.  A word counts only when it carries exactly seq, so the workspace may start with any contents,
// and a graph replay (which repeats seq) finds the words zeroed.  With zero_counters, block 0 also
// zeroes the counters and the error word of the one-launch decode experts path that follows
// (sync[0, kSyncCounters)).
template <int MAXJ, int NT, int G>
__global__ __launch_bounds__(512) void k_route_small(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, float* __restrict__ logits,
    const float* __restrict__ bias, int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ zero_w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ inv_perm, int32_t* __restrict__ sync, unsigned long long* __restrict__ tagged,
    int zero_counters, int seq, int N, int H, int R, int E, int K, int scoring, int renorm, float scale) {
  __shared__ float p_lds[8][MAXJ * 64];
  __shared__ int s_ids[64];
  __shared__ int s_off[1024];
  __shared__ int s_expired;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r = blockIdx.x * 8 + wave;
  if (r < R) {  // wave-uniform
    float acc[NT];
    gemv_column<NT, G>(x, wr, N, H, r, acc);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < N) {  // uniform
        const float v = wave_sum(acc[t]);
        if (lane == 0)
          __hip_atomic_store(tagged + (size_t)t * R + r, ((unsigned long long)(uint32_t)seq << 32) | __float_as_uint(v),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (blockIdx.x != 0) return;  // block 0 waits for the tagged logits themselves
  if (tid == 0) s_expired = 0;
  for (int i = tid; i < R; i += 512) s_off[i] = 0;
  if (zero_counters)
    for (int i = tid; i < kSyncCounters; i += 512) sync[i] = 0;
  __syncthreads();
  if (wave < N) {
    const int my_id = topk_token<MAXJ, true>(reinterpret_cast<const float*>(tagged), 1, logits, bias, ids, w, zero_w,
                                             p_lds[wave], wave, N, R, E, K, scoring, renorm, scale, (uint32_t)seq,
                                             &s_expired);
    if (lane < K) s_ids[wave * K + lane] = my_id;
  }
  __syncthreads();
  if (tid == 0 && s_expired)  // after the zeroing above: this launch's output is undefined
    __hip_atomic_store(sync + kSyncError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (wave == 0) sort_rows_ballot(s_ids, s_off, N * K, R, counts, offsets, sorted_ids, inv_perm);
}

bool route_small_fits(int N, int K, int R) { return N <= RG_MAXN && N * K <= kWave && R <= 1024; }

hipError_t launch_route_small(const uint16_t* x, const uint16_t* router_w, float* logits, const float* bias,
                              int32_t* ids, float* w, float* zero_w, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_ids, int32_t* inv_perm, int32_t* sync, unsigned long long* tagged,
                              bool zero_counters, int seq, int N, int H, int R, int E, int K, int scoring,
                              int renormalize, float routed_scale, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (!route_small_fits(N, K, R) || seq == 0) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((R + 7) / 8);
  const int maxj = (R + 63) / 64;
#define MOE_ROUTE_CASE(J)                                                                                        \
  case J:                                                                                                        \
    if (N <= 4)                                                                                                  \
      k_route_small<J, 4, 4><<<blocks, 512, 0, s>>>(x, router_w, logits, bias, ids, w, zero_w, counts, offsets,  \
                                                    sorted_ids, inv_perm, sync, tagged, zero_counters, seq, N, H, \
                                                    R, E, K, scoring, renormalize, routed_scale);                 \
    else                                                                                                         \
      k_route_small<J, 8, 2><<<blocks, 512, 0, s>>>(x, router_w, logits, bias, ids, w, zero_w, counts, offsets,  \
                                                    sorted_ids, inv_perm, sync, tagged, zero_counters, seq, N, H, \
                                                    R, E, K, scoring, renormalize, routed_scale);                 \
    break;
  switch (maxj <= 2 ? maxj : (maxj <= 4 ? 4 : (maxj <= 6 ? 6 : 16))) {
    MOE_ROUTE_CASE(1)
    MOE_ROUTE_CASE(2)
    MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(6)
    MOE_ROUTE_CASE(16)
  }
#undef MOE_ROUTE_CASE
  return hipGetLastError();
}

int router_slices(int N, int H, int R, bool row_invariant) {
  if (row_invariant) {  // a function of H only: the largest power of two <= 16 dividing H / 128
    int S = 1;
    while (S < 16 && (H / 128) % (2 * S) == 0) S *= 2;
    return S;
  }
  if (N <= RG_MAXN) return 1;  // the GEMV router writes whole logits
  const long tiles = (long)((N + RT_BM - 1) / RT_BM) * ((R + RT_BN - 1) / RT_BN);
  int S = 1;
  while (tiles * S < 1024 && S < 16 && (H / 128) % (2 * S) == 0) S *= 2;  // topk adds at most 16 planes
  return S;
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* router_w, float* part, int N, int H, int R,
                                int slices, bool row_invariant, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (N <= RG_MAXN && !row_invariant) {
    const unsigned blocks = (unsigned)((R + 3) / 4);
    if (N <= 4) k_router_gemv<4, 4><<<blocks, 256, 0, s>>>(x, router_w, part, N, H, R);
    else k_router_gemv<8, 2><<<blocks, 256, 0, s>>>(x, router_w, part, N, H, R);
    return hipGetLastError();
  }
  dim3 grid((N + RT_BM - 1) / RT_BM, (R + RT_BN - 1) / RT_BN, slices);
  k_router_logits<<<grid, 256, 0, s>>>(x, router_w, part, N, H, R, H / slices);
  return hipGetLastError();
}

hipError_t launch_topk(const float* part, int slices, float* logits, const float* bias, int32_t* ids, float* w,
                       float* zero_w, int N, int R, int E, int K, int scoring, int renormalize, float routed_scale,
                       hipStream_t s) {
  if (N == 0) return hipSuccess;
  dim3 grid((N + 3) / 4), block(256);
  const int maxj = (R + 63) / 64;
#define MOE_TOPK_CASE(J)                                                                                      \
  case J:                                                                                                     \
    k_topk<J><<<grid, block, 0, s>>>(part, slices, logits, bias, ids, w, zero_w, N, R, E, K, scoring,        \
                                     renormalize, routed_scale);                                              \
    break;
  switch (maxj <= 6 ? maxj : (maxj <= 8 ? 8 : 16)) {
    MOE_TOPK_CASE(1)
    MOE_TOPK_CASE(2)
    MOE_TOPK_CASE(3)
    MOE_TOPK_CASE(4)
    MOE_TOPK_CASE(5)
    MOE_TOPK_CASE(6)
    MOE_TOPK_CASE(8)
    MOE_TOPK_CASE(16)
  }
#undef MOE_TOPK_CASE
  return hipGetLastError();
}

bool topk_sort_small_fits(int N, int K) { return N <= 64 && N * K <= 1024; }

hipError_t launch_topk_sort_small(const float* part, int slices, float* logits, const float* bias, int32_t* ids,
                                  float* w, float* zero_w, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                                  int32_t* inv_perm, int32_t* done, int done_len, int N, int R, int E, int K,
                                  int scoring, int renormalize, float routed_scale, hipStream_t s) {
  if (N == 0) return hipSuccess;
  const int maxj = (R + 63) / 64;
#define MOE_SMALL_CASE(J)                                                                                      \
  case J:                                                                                                      \
    k_topk_sort_small<J><<<1, 1024, 0, s>>>(part, slices, logits, bias, ids, w, zero_w, counts, offsets,        \
                                            sorted_ids, inv_perm, done, done_len, N, R, E, K, scoring,            \
                                            renormalize, routed_scale);                                          \
    break;
  switch (maxj <= 2 ? maxj : (maxj <= 4 ? 4 : (maxj <= 6 ? 6 : 16))) {
    MOE_SMALL_CASE(1)
    MOE_SMALL_CASE(2)
    MOE_SMALL_CASE(4)
    MOE_SMALL_CASE(6)
    MOE_SMALL_CASE(16)
  }
#undef MOE_SMALL_CASE
  return hipGetLastError();
}

}  // namespace moe
