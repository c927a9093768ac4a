// Launch functions of the gfx950 MoE kernels (internal to libmoe; the C ABI in
// include/moe.h validates arguments before calling these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Raise a kernel's dynamic LDS limit to `bytes` on the current device, once per (kernel, device);
// thread-safe.  Kernels that use more than the default dynamic LDS call this before each launch.
hipError_t ensure_dynamic_lds(const void* kernel, int bytes);
// compute units of the current device, looked up once per device (0 if it cannot be queried)
int device_cus();

// a1 + a2: router logits (split over `slices` parts of H, each writing an [N, R]
// partial plane) and top-K selection (adds the planes in order; when slices > 1
// it also writes the summed logits to `logits`)
// row_invariant: the MFMA kernel at every N with a split that depends on H only (no GEMV)
int router_slices(int N, int H, int R, bool row_invariant);
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* router_w, float* part, int N, int H, int R,
                                int slices, bool row_invariant, hipStream_t s);
hipError_t launch_topk(const float* part, int slices, float* logits, const float* bias, int32_t* ids, float* w,
                       float* zero_w, int N, int R, int E, int K, int scoring, int renormalize, float routed_scale,
                       hipStream_t s);

// a2 + a3 for small batches (N <= 64, N*K <= 1024): top-K and the stable sort in one block
bool topk_sort_small_fits(int N, int K);
// `done` ([done_len] int32, may be null) is zeroed for a following one-launch decode (its counters and
// its error word)
hipError_t launch_topk_sort_small(const float* part, int slices, float* logits, const float* bias, int32_t* ids,
                                  float* w, float* zero_w, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                                  int32_t* inv_perm, int32_t* done, int done_len, int N, int R, int E, int K,
                                  int scoring, int renormalize, float routed_scale, hipStream_t s);

// a1 + a2 + a3 for decode batches (route_small_fits: N <= 8, N*K <= 64, R <= 1024, not row-invariant):
// router GEMV, top-K and the sort in one launch, with the same results as launch_router_logits (one
// slice) + launch_topk_sort_small.  tagged: N R 64-bit words of scratch (any contents but `seq` in a
// high half) through which the GEMV blocks hand the logits to the top-K block; the launch leaves them
// zero.  seq: nonzero, different from the last launch's on these words.  sync: the workspace's sync
// piece (kSyncInts int32), whose error word is set if the top-K block's bounded wait expires.
// zero_counters: also zero sync[0, kSyncCounters) for a following one-launch decode.
bool route_small_fits(int N, int K, int R);
hipError_t launch_route_small(const uint16_t* x, const uint16_t* router_w, float* logits, const float* bias,
                              int32_t* ids, float* w, float* zero_w, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_ids, int32_t* inv_perm, int32_t* sync, unsigned long long* tagged,
                              bool zero_counters, int seq, int N, int H, int R, int E, int K, int scoring,
                              int renormalize, float routed_scale, hipStream_t s);

// a3: stable counting sort by expert; hist is [(permute_chunks(P) + 1) * 4 ceil(R / 4)] int32 scratch.  Two
// launches when permute_direct(P, R), else three.  clear8 (or null): 8 ints that the sort sets to zero (the
// tile counters of the GEMMs after it).
int permute_chunks(int P);
bool permute_direct(int P, int R);
hipError_t launch_permute(const int32_t* ids, int P, int R, int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                          int32_t* inv_perm, int32_t* hist, int32_t* clear8, hipStream_t s);

// a4: per-token, per-128-column e4m3 quantisation of bf16 rows
hipError_t launch_quant_fp8(const uint16_t* x, uint8_t* xq, float* xs, int rows, int cols, hipStream_t s);

// a5 / a6: grouped expert GEMMs
struct GroupedGemmArgs {
  int stage;   // 0: gate/up + SwiGLU, 1: down
  int shared;  // 1: only the shared expert, over all N rows (identity row map, direct weights)
  int with_shared;  // 1: the routed experts and, as one more group (index E), the shared expert
  int N, H, I, K, E;  // I: the routed experts' intermediate size (the shared one's when `shared`)
  int Is;             // the shared expert's intermediate size (with_shared or shared)
  int P;               // N*K (routed) or N (shared): upper bound of rows
  const void* a;        // gate/up: x [N,H] (bf16 or e4m3); down: h [rows, I]
  const float* a_scales;  // fp8 only
  const int32_t* sorted_ids;  // routed only
  const int32_t* offsets;     // routed only: [E+1] (only the first E+1 entries are read)
  const void* const* w_gate;  // routed: device tables; shared: nullptr
  const void* const* w_up;
  const void* const* w_down;
  const float* const* s_gate;
  const float* const* s_up;
  const float* const* s_down;
  const void* sh_gate;  // shared: direct pointers
  const void* sh_up;
  const void* sh_down;
  const float* sh_gate_s;
  const float* sh_up_s;
  const float* sh_down_s;
  void* out;           // gate/up: h [rows, I] (bf16 or e4m3); down: y [rows, H] bf16
  float* out_scales;   // fp8 gate/up only: [rows, I/128]
  // the shared group's operands (shared or with_shared): A rows are tokens (gate/up: x, as `a`; down:
  // its h [N, Is]), outputs at the token's row (gate/up: h [N, Is]; down: y [N, H])
  const void* sh_a;
  const float* sh_a_scales;
  void* sh_out;
  float* sh_out_scales;
  int row_invariant;   // 1: only the kernels whose per-row arithmetic is the same at any row count
  // Splitting the last, partial round of tiles along K (bf16 tile kernel): `slots` blocks of the kernel
  // fit on the GPU at once (0: never split); split_part holds the parts' fp32 partial sums
  // (kSplitSlots x kSplitFloats) and split_cnt their arrival counters (kSyncSplitMax 64-bit words, any
  // contents: a word counts only while its high half holds split_seq, a nonzero value of this launch
  // that differs from the previous launch's; the last part of a tile puts its word back to 0).
  int slots;
  uint32_t split_seq;
  float* split_part;
  unsigned long long* split_cnt;
  // Tiles handed out at run time (the MXFP4 persistent down kernel; other kernels ignore it): 8 counters,
  // one per XCD, holding zero when the launch starts (a launch that takes them leaves them zero), or null
  // (a fixed walk).
  int32_t* queue;
};
// Limits of the K split: at most kSplitParts parts per tile, kSplitSlots parts per launch, each part's
// partial tile kSplitFloats fp32 (256 threads x 128 accumulators).
constexpr int kSplitParts = 4, kSplitSlots = 512, kSplitFloats = 256 * 128;
hipError_t launch_grouped_gemm_bf16(const GroupedGemmArgs& g, hipStream_t s);
// bf16 streaming kernel for a few rows per expert (decode)
bool decode_gemm_fits(const GroupedGemmArgs& g);
hipError_t launch_grouped_gemm_decode(const GroupedGemmArgs& g, hipStream_t s);
// Operands of the unpermute-reduce step (see launch_unpermute_reduce).
struct ReduceArgs {
  const int32_t* inv_perm;   // [N, K] sorted row of each (token, slot)
  const int32_t* ids;        // [N, K] expert ids (>= E: identity expert)
  const float* w;            // [N, K] routing weights
  const uint16_t* x;         // [N, H] layer input (identity experts)
  const uint16_t* shared_y;  // [N, H] shared expert output or null
  const uint16_t* shared_gate;  // [H] bf16 sigmoid gate row of the shared expert, or null (weight 1)
  uint16_t* out;             // [N, H]
  int N, H, K, E;
};
// The counters of the one-launch decode path: kSyncInts int32 at a fixed place (the start of the
// workspace), whose indices do not depend on the layer's sizes, so that a workspace reused for
// another batch size finds them where the last call left them.
constexpr int kSyncExperts = 0;         // [1024]: gate/up tiles finished, per expert
constexpr int kSyncColTiles = 1024;     // [kSyncMaxColTiles]: down tiles finished, per 128-column block
constexpr int kSyncMaxColTiles = 512;   // so the path takes H <= 65536
constexpr int kSyncReduced = 1536;      // column blocks reduced
constexpr int kSyncError = 1537;        // set to 1 when a bounded wait expires; the launch never clears it
constexpr int kSyncCounters = 1538;     // sync[0, kSyncCounters): the counters above and the error word
constexpr int kSyncSplit = kSyncCounters;  // [kSyncSplitMax] 64-bit: split tiles' arrivals
constexpr int kSyncSplitMax = kSplitSlots / 2;                     // a split tile has at least two parts
constexpr int kSyncQueue = kSyncSplit + 2 * kSyncSplitMax;  // [8]: per-XCD tile counters of a launch
constexpr int kSyncInts = kSyncQueue + 8;
static_assert(kSyncSplit % 2 == 0, "64-bit counters");
// Routed gate/up, down and the unpermute-reduce of a decode layer in one launch (the shared expert,
// if any, must already be in r.shared_y).  sync: kSyncInts int32 whose counters hold zeros when the
// launch starts; the launch leaves them zero (and sets sync[kSyncError] if a wait expired).
bool decode_fused_fits(int E, int H);
hipError_t launch_decode_fused(const GroupedGemmArgs& gu, const GroupedGemmArgs& dn, const ReduceArgs& r,
                               int32_t* sync, hipStream_t s);

hipError_t launch_grouped_gemm_fp8(const GroupedGemmArgs& g, hipStream_t s);
// whether launch_grouped_gemm_fp8 takes the streaming kernel for g (else the register-staged one)
bool fp8_streams(const GroupedGemmArgs& g);
// MXFP4 weights (packed E2M1 [rows, K/2], E8M0 scales [rows, K/32] in the s_* / sh_*_s pointers)
hipError_t launch_grouped_gemm_mxfp4(const GroupedGemmArgs& g, hipStream_t s);

// unpermute + weighted reduce + identity-expert and (gated) shared blends
hipError_t launch_unpermute_reduce(const uint16_t* y_sorted, const ReduceArgs& r, hipStream_t s);

}  // namespace moe
