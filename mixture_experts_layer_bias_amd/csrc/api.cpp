// The C ABI of libmoe (declared and documented in include/moe.h): argument
// validation, the workspace layout and the launch sequence of moe_forward.
// Host code only; every launch goes to the caller's stream and nothing here
// allocates or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <random>
#include <algorithm>
#include <map>
#include <set>
#include <utility>

#include "kernels.h"
#include "moe.h"

namespace moe {

// Compute units of the current device (looked up once per device); 0 if it cannot be queried.
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> per_device;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = per_device.find(dev);
  if (it != per_device.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
  per_device[dev] = cus;
  return cus;
}

hipError_t ensure_dynamic_lds(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;  // (kernel, device)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kernel, dev})) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({kernel, dev});
  return e;
}

}  // namespace moe

namespace {

thread_local char g_err[512] = "";

// A nonzero value per launch of the one-launch decode prelude, different from the previous launch's
// (a process-wide counter from a random start, so a workspace's leftover flags are not mistaken for it).
int next_route_seq() {
  static std::atomic<uint32_t> ctr{std::random_device{}()};
  for (;;) {
    const uint32_t v = ctr.fetch_add(1, std::memory_order_relaxed) + 1u;
    if (v != 0) return (int)v;
  }
}

// A nonzero value per launch of the bf16 tile kernel that may split tiles along K, different from the
// previous launch's (its arrival counters count only words tagged with it).
uint32_t next_split_seq() {
  static std::atomic<uint32_t> ctr{std::random_device{}()};
  for (;;) {
    const uint32_t v = ctr.fetch_add(1, std::memory_order_relaxed) + 1u;
    if (v != 0) return v;
  }
}


// Blocks of the bf16 tile kernel (two per compute unit) that the current device holds at once, a
// multiple of 8 and at most kSplitSlots; 0 if the device cannot be queried.
int split_slots() { return std::min(2 * ::moe::device_cus(), moe::kSplitSlots) / 8 * 8; }

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

moe_status_t ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

#define MOE_CHECK(cond, st, ...) \
  do {                           \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define MOE_HIP(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

#define MOE_RET(expr)                   \
  do {                                  \
    moe_status_t s_ = (expr);           \
    if (s_ != MOE_OK) return s_;        \
  } while (0)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status_t check_ptr(const void* p, size_t align, const char* name) {
  MOE_CHECK(p != nullptr, MOE_ERR_INVALID, "%s is NULL", name);
  MOE_CHECK(aligned(p, align), MOE_ERR_INVALID, "%s is not %zu-byte aligned", name, align);
  return MOE_OK;
}

moe_status_t check_config(const moe_config_t* c) {
  MOE_CHECK(c != nullptr, MOE_ERR_INVALID, "config is NULL");
  MOE_CHECK(c->num_tokens >= 0, MOE_ERR_INVALID, "num_tokens %d < 0", c->num_tokens);
  MOE_CHECK(c->num_experts >= 1, MOE_ERR_INVALID, "num_experts %d < 1", c->num_experts);
  MOE_CHECK(c->router_width >= c->num_experts, MOE_ERR_INVALID, "router_width %d < num_experts %d",
            c->router_width, c->num_experts);
  MOE_CHECK(c->top_k >= 1 && c->top_k <= c->router_width, MOE_ERR_INVALID, "top_k %d not in [1, router_width %d]",
            c->top_k, c->router_width);
  MOE_CHECK(c->scoring == MOE_SCORING_SOFTMAX || c->scoring == MOE_SCORING_SIGMOID ||
                c->scoring == MOE_SCORING_SQRTSOFTPLUS,
            MOE_ERR_INVALID, "scoring %d is not a MOE_SCORING_* value", c->scoring);
  MOE_CHECK(c->weight_dtype == MOE_WEIGHTS_BF16 || c->weight_dtype == MOE_WEIGHTS_FP8_E4M3 ||
                c->weight_dtype == MOE_WEIGHTS_MXFP4,
            MOE_ERR_INVALID,
            "weight_dtype %d is not a MOE_WEIGHTS_* value", c->weight_dtype);
  MOE_CHECK(std::isfinite(c->routed_scale), MOE_ERR_INVALID, "routed_scale is not finite");
  MOE_CHECK(c->row_invariant == 0 || c->row_invariant == 1, MOE_ERR_INVALID, "row_invariant %d is not 0 or 1",
            c->row_invariant);
  MOE_CHECK(c->hidden > 0 && c->inter > 0 && c->shared_inter >= 0, MOE_ERR_INVALID,
            "hidden %d, inter %d must be > 0 and shared_inter %d >= 0", c->hidden, c->inter, c->shared_inter);
  MOE_CHECK(c->router_width <= 1024, MOE_ERR_UNSUPPORTED, "router_width %d > 1024", c->router_width);
  MOE_CHECK(c->top_k <= 32, MOE_ERR_UNSUPPORTED, "top_k %d > 32", c->top_k);
  MOE_CHECK(c->hidden % 128 == 0, MOE_ERR_UNSUPPORTED, "hidden %d is not a multiple of 128", c->hidden);
  MOE_CHECK(c->inter % 128 == 0, MOE_ERR_UNSUPPORTED, "inter %d is not a multiple of 128", c->inter);
  MOE_CHECK(c->shared_inter % 128 == 0, MOE_ERR_UNSUPPORTED, "shared_inter %d is not a multiple of 128",
            c->shared_inter);
  MOE_CHECK((int64_t)c->num_tokens * c->top_k < (int64_t)1 << 30, MOE_ERR_UNSUPPORTED,
            "num_tokens * top_k = %lld is too large", (long long)c->num_tokens * c->top_k);
  return MOE_OK;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Whether the layer's bf16 tile-kernel launches may split their last round of tiles along K (and so
// need the `split` piece): bf16 weights, not row-invariant, no shared expert (whose launches, folded or
// not, then keep the bits of moe_forward's), launches of at least 2048 routed rows, and a GEMM with K of at
// least 4096 (H for gate/up, I for down; see with_split).
bool uses_split(const moe_config_t* c) {
  return c->weight_dtype == MOE_WEIGHTS_BF16 && c->row_invariant == 0 && c->shared_inter == 0 &&
         (int64_t)c->num_tokens * c->top_k >= 2048 && (c->hidden >= 4096 || c->inter >= 4096);
}

void compute_layout(const moe_config_t* c, moe_workspace_layout_t* L) {
  const size_t N = c->num_tokens, H = c->hidden, R = c->router_width, K = c->top_k, I = c->inter,
               Is = c->shared_inter, P = N * K;
  const bool fp8 = c->weight_dtype != MOE_WEIGHTS_BF16;  // fp8 or mxfp4: e4m3 activations, scaled weights
  const size_t none = SIZE_MAX;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  // first, at a place and size independent of the layer's sizes: the one-launch decode path's
  // counters stay where the previous call left them (zero) whatever the batch size
  L->sync = take((size_t)moe::kSyncInts * 4);
  L->sync_error = L->sync + (size_t)moe::kSyncError * 4;
  L->logits = take(N * R * 4);
  L->topk_ids = take(P * 4);
  L->topk_w = take(P * 4);
  L->zero_w = take(N * 4);
  L->counts = take(R * 4);
  L->offsets = take((R + 1) * 4);
  L->sorted_ids = take(P * 4);
  L->inv_perm = take(P * 4);
  const int slices = moe::router_slices((int)N, (int)H, (int)R, c->row_invariant != 0);
  // chunk histograms (rows padded to 4 ints) + bucket totals
  const size_t hist_bytes = ((size_t)moe::permute_chunks((int)P) + 1) * ((R + 3) / 4 * 4) * 4;
  const size_t part_bytes = slices > 1 ? (size_t)slices * N * R * 4 : 0;
  // a decode batch's one-launch routing hands the logits over as 64-bit tagged words
  const size_t tag_bytes = moe::route_small_fits((int)N, (int)K, (int)R) ? N * R * 8 : 0;
  L->scratch = take(std::max(hist_bytes, std::max(part_bytes, tag_bytes)));
  L->xq = fp8 ? take(N * H) : none;
  L->x_scales = fp8 ? take(N * (H / 128) * 4) : none;
  L->h = take(P * I * (fp8 ? 1 : 2));
  L->h_scales = fp8 ? take(P * (I / 128) * 4) : none;
  L->y = take(P * H * 2);
  L->shared_h = Is ? take(N * Is * (fp8 ? 1 : 2)) : none;
  L->shared_h_scales = (Is && fp8) ? take(N * (Is / 128) * 4) : none;
  L->shared_y = Is ? take(N * H * 2) : none;
  L->split = uses_split(c) ? take((size_t)moe::kSplitSlots * moe::kSplitFloats * 4) : none;
  L->total = off;
}

moe_status_t check_weights(const moe_config_t* c, const moe_weights_t* w) {
  MOE_CHECK(w != nullptr, MOE_ERR_INVALID, "weights is NULL");
  MOE_RET(check_ptr(w->router_w, 16, "router_w"));
  if (w->correction_bias) MOE_RET(check_ptr(w->correction_bias, 4, "correction_bias"));
  MOE_RET(check_ptr(w->gate_w, 8, "gate_w table"));
  MOE_RET(check_ptr(w->up_w, 8, "up_w table"));
  MOE_RET(check_ptr(w->down_w, 8, "down_w table"));
  const bool fp8 = c->weight_dtype != MOE_WEIGHTS_BF16;  // fp8 or mxfp4: e4m3 activations, scaled weights
  if (fp8) {
    MOE_RET(check_ptr(w->gate_s, 8, "gate_s table"));
    MOE_RET(check_ptr(w->up_s, 8, "up_s table"));
    MOE_RET(check_ptr(w->down_s, 8, "down_s table"));
  }
  if (c->shared_inter > 0) {
    MOE_RET(check_ptr(w->sh_gate_w, 16, "sh_gate_w"));
    MOE_RET(check_ptr(w->sh_up_w, 16, "sh_up_w"));
    MOE_RET(check_ptr(w->sh_down_w, 16, "sh_down_w"));
    if (fp8) {
      MOE_RET(check_ptr(w->sh_gate_s, 4, "sh_gate_s"));
      MOE_RET(check_ptr(w->sh_up_s, 4, "sh_up_s"));
      MOE_RET(check_ptr(w->sh_down_s, 4, "sh_down_s"));
    }
    if (w->sh_expert_gate) MOE_RET(check_ptr(w->sh_expert_gate, 16, "sh_expert_gate"));
  } else {
    MOE_CHECK(w->sh_expert_gate == nullptr, MOE_ERR_INVALID, "sh_expert_gate is set but shared_inter is 0");
  }
  return MOE_OK;
}

moe::GroupedGemmArgs gemm_args(const moe_config_t* c, int stage, int group, const moe_weights_t* w, const void* a,
                               const float* a_scales, const int32_t* sorted_ids, const int32_t* offsets, void* out,
                               float* out_scales) {
  moe::GroupedGemmArgs g{};
  g.stage = stage;
  g.shared = group == MOE_GROUP_SHARED;
  g.with_shared = 0;
  g.N = c->num_tokens;
  g.H = c->hidden;
  g.I = g.shared ? c->shared_inter : c->inter;
  g.Is = c->shared_inter;
  g.K = c->top_k;
  g.E = c->num_experts;
  g.P = g.shared ? c->num_tokens : c->num_tokens * c->top_k;
  g.a = a;
  g.a_scales = a_scales;
  g.sorted_ids = sorted_ids;
  g.offsets = offsets;
  g.w_gate = w->gate_w;
  g.w_up = w->up_w;
  g.w_down = w->down_w;
  g.s_gate = w->gate_s;
  g.s_up = w->up_s;
  g.s_down = w->down_s;
  g.sh_gate = w->sh_gate_w;
  g.sh_up = w->sh_up_w;
  g.sh_down = w->sh_down_w;
  g.sh_gate_s = w->sh_gate_s;
  g.sh_up_s = w->sh_up_s;
  g.sh_down_s = w->sh_down_s;
  g.out = out;
  g.out_scales = out_scales;
  if (g.shared) {  // the shared group reads and writes through the sh_* operands
    g.sh_a = a;
    g.sh_a_scales = a_scales;
    g.sh_out = out;
    g.sh_out_scales = out_scales;
  }
  g.row_invariant = c->row_invariant;
  return g;
}

// The routed launch `routed` with the shared expert carried as one more group (index E): its A rows
// are tokens of `sh_a`, its output rows go to `sh_out`.
moe::GroupedGemmArgs with_shared(moe::GroupedGemmArgs routed, const void* sh_a, const float* sh_a_scales,
                                 void* sh_out, float* sh_out_scales) {
  routed.with_shared = 1;
  routed.sh_a = sh_a;
  routed.sh_a_scales = sh_a_scales;
  routed.sh_out = sh_out;
  routed.sh_out_scales = sh_out_scales;
  return routed;
}

// The shared expert rides in the routed launch of a stage as one more group when the tile schedulers'
// group tables have room for it and that launch takes the kernel that the routed experts and the
// shared expert would each take in a launch of their own (so every output keeps its bits).
constexpr int kMaxLaunchGroups = 1024;
bool same_kernel(const moe_config_t* c, const moe::GroupedGemmArgs& routed, const moe::GroupedGemmArgs& shared) {
  if (c->weight_dtype == MOE_WEIGHTS_BF16) return moe::decode_gemm_fits(routed) == moe::decode_gemm_fits(shared);
  if (c->weight_dtype == MOE_WEIGHTS_FP8_E4M3) return moe::fp8_streams(routed) == moe::fp8_streams(shared);
  return true;  // MXFP4: one kernel pair
}
bool fold_shared(const moe_config_t* c, int stage) {
  if (c->shared_inter <= 0 || c->num_experts + 1 > kMaxLaunchGroups) return false;
  const moe_weights_t none{};  // the kernel choice is a function of the sizes only
  return same_kernel(c, gemm_args(c, stage, MOE_GROUP_ROUTED, &none, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
                     gemm_args(c, stage, MOE_GROUP_SHARED, &none, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr));
}

// Let a routed launch split its last round of tiles along K, with the workspace's `split` piece and
// arrival counters (a no-op for a layer without that piece).  Only launches whose tiles are long (K of at
// least 4096) split: there the last round, a tile-time long, costs most (measured: zero-computation-
// expert layer gate/up, K 6144, 666 -> 617 us); shorter tiles gained nothing, and every launch that
// may split carries `slots` more blocks, which only find that they have nothing to do.
moe::GroupedGemmArgs with_split(moe::GroupedGemmArgs g, const moe_workspace_layout_t& L, char* base) {
  if (L.split == SIZE_MAX || g.shared || g.with_shared) return g;
  if ((g.stage == 0 ? g.H : g.I) < 4096) return g;
  g.slots = split_slots();
  g.split_seq = next_split_seq();
  g.split_part = reinterpret_cast<float*>(base + L.split);
  g.split_cnt = reinterpret_cast<unsigned long long*>(base + L.sync + (size_t)moe::kSyncSplit * 4);
  return g;
}

moe_status_t run_gemm(const moe_config_t* c, const moe::GroupedGemmArgs& g, hipStream_t s) {
  if (c->weight_dtype == MOE_WEIGHTS_BF16) {
    MOE_HIP(moe::launch_grouped_gemm_bf16(g, s));
  } else if (c->weight_dtype == MOE_WEIGHTS_FP8_E4M3) {
    MOE_HIP(moe::launch_grouped_gemm_fp8(g, s));
  } else {
    MOE_HIP(moe::launch_grouped_gemm_mxfp4(g, s));
  }
  return MOE_OK;
}

// Whether the decode experts path (routed gate/up, down and the reduce in one launch, with the shared
// expert as one more group when it folds) applies.
bool experts_fused(const moe_config_t* c) {
  if (c->weight_dtype != MOE_WEIGHTS_BF16 || c->row_invariant) return false;
  if (c->shared_inter > 0 && !(fold_shared(c, MOE_STAGE_GATE_UP) && fold_shared(c, MOE_STAGE_DOWN))) return false;
  if (!moe::decode_fused_fits(c->num_experts + (c->shared_inter > 0 ? 1 : 0), c->hidden)) return false;
  const moe_weights_t none{};  // the fit is a function of the sizes only
  moe::GroupedGemmArgs gu = gemm_args(c, MOE_STAGE_GATE_UP, MOE_GROUP_ROUTED, &none, nullptr, nullptr, nullptr,
                                      nullptr, nullptr, nullptr);
  moe::GroupedGemmArgs dn = gemm_args(c, MOE_STAGE_DOWN, MOE_GROUP_ROUTED, &none, nullptr, nullptr, nullptr, nullptr,
                                      nullptr, nullptr);
  if (c->shared_inter > 0) {
    gu = with_shared(gu, nullptr, nullptr, nullptr, nullptr);
    dn = with_shared(dn, nullptr, nullptr, nullptr, nullptr);
  }
  return moe::decode_gemm_fits(gu) && moe::decode_gemm_fits(dn);
}

// The expert half of the layer given the routing: [quantise] -> gate/up (+ shared) -> down
// (+ shared) -> unpermute-reduce.  With `fused` (the counters piece of the workspace holds zeros)
// the routed GEMMs and the reduce run as one launch, after the shared expert, whose output the
// reduce reads; that launch leaves the counters zero again.
// queue: the workspace's per-XCD tile counters, zero (or null: the launches walk their tiles in a fixed order)
moe_status_t run_experts(const moe_config_t* cfg, const moe_weights_t* w, const void* x, const int32_t* ids,
                         const float* tw, const int32_t* offsets, const int32_t* sorted_ids, const int32_t* inv_perm,
                         void* out, const moe_workspace_layout_t& L, char* base, bool fused, int32_t* queue,
                         hipStream_t s) {
  const moe_config_t& c = *cfg;
  auto at = [&](size_t off) -> void* { return off == SIZE_MAX ? nullptr : base + off; };
  const bool fp8 = c.weight_dtype != MOE_WEIGHTS_BF16;  // e4m3 activations
  if (fp8)
    MOE_HIP(moe::launch_quant_fp8(static_cast<const uint16_t*>(x), static_cast<uint8_t*>(at(L.xq)),
                                  static_cast<float*>(at(L.x_scales)), c.num_tokens, c.hidden, s));
  const void* a = fp8 ? at(L.xq) : x;
  const float* a_scales = fp8 ? static_cast<const float*>(at(L.x_scales)) : nullptr;
  const moe::GroupedGemmArgs gu = gemm_args(cfg, MOE_STAGE_GATE_UP, MOE_GROUP_ROUTED, w, a, a_scales, sorted_ids,
                                            offsets, at(L.h), static_cast<float*>(at(L.h_scales)));
  const moe::GroupedGemmArgs dn = gemm_args(cfg, MOE_STAGE_DOWN, MOE_GROUP_ROUTED, w, at(L.h),
                                            static_cast<float*>(at(L.h_scales)), sorted_ids, offsets, at(L.y), nullptr);
  const moe::GroupedGemmArgs sh_gu = gemm_args(cfg, MOE_STAGE_GATE_UP, MOE_GROUP_SHARED, w, a, a_scales, nullptr,
                                               nullptr, at(L.shared_h), static_cast<float*>(at(L.shared_h_scales)));
  const moe::GroupedGemmArgs sh_dn = gemm_args(cfg, MOE_STAGE_DOWN, MOE_GROUP_SHARED, w, at(L.shared_h),
                                               static_cast<float*>(at(L.shared_h_scales)), nullptr, nullptr,
                                               at(L.shared_y), nullptr);
  const moe::ReduceArgs red{inv_perm,
                            ids,
                            tw,
                            static_cast<const uint16_t*>(x),
                            static_cast<const uint16_t*>(at(L.shared_y)),
                            c.shared_inter > 0 ? static_cast<const uint16_t*>(w->sh_expert_gate) : nullptr,
                            static_cast<uint16_t*>(out),
                            c.num_tokens,
                            c.hidden,
                            c.top_k,
                            c.num_experts};
  // the shared expert as one more group of the routed launches (same per-row arithmetic as its own
  // launches), or, when the group tables have no room for it, in launches of its own
  const bool fold_gu = fold_shared(cfg, MOE_STAGE_GATE_UP), fold_dn = fold_shared(cfg, MOE_STAGE_DOWN);
  const moe::GroupedGemmArgs gu_all =
      fold_gu ? with_shared(gu, a, a_scales, at(L.shared_h), static_cast<float*>(at(L.shared_h_scales))) : gu;
  const moe::GroupedGemmArgs dn_all =
      fold_dn ? with_shared(dn, at(L.shared_h), static_cast<float*>(at(L.shared_h_scales)), at(L.shared_y), nullptr)
              : dn;
  if (fused) {  // implies both folds when there is a shared expert
    MOE_HIP(moe::launch_decode_fused(gu_all, dn_all, red, static_cast<int32_t*>(at(L.sync)), s));
    return ok();
  }
  auto queued = [&](moe::GroupedGemmArgs g) {
    g.queue = queue;
    return g;
  };
  MOE_RET(run_gemm(cfg, with_split(queued(gu_all), L, base), s));
  if (c.shared_inter > 0 && !fold_gu) MOE_RET(run_gemm(cfg, queued(sh_gu), s));
  MOE_RET(run_gemm(cfg, with_split(queued(dn_all), L, base), s));
  if (c.shared_inter > 0 && !fold_dn) MOE_RET(run_gemm(cfg, queued(sh_dn), s));
  MOE_HIP(moe::launch_unpermute_reduce(static_cast<const uint16_t*>(at(L.y)), red, s));
  return ok();
}

// ---- the workspace of moe_forward_noalloc: one array in the library's code object, so each GPU the
// library runs on holds its own copy from load until the process ends.  In host code `scratch` names
// a host-side stand-in, never the device memory: kernels get the address that hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, looked up once

// The address of `scratch` on the current device (looked up at the first call on that device, with it
// current).
moe_status_t scratch_on_current_device(void** ptr) {
  int dev = 0;
  MOE_HIP(hipGetDevice(&dev));
  MOE_CHECK(dev >= 0 && dev < kMaxDevices, MOE_ERR_UNSUPPORTED, "device %d: only devices 0..%d are supported", dev,
            kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    MOE_CHECK(p != nullptr && aligned(p, 256), MOE_ERR_HIP, "static workspace of device %d has no usable address",
              dev);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

moe_status_t launch_route(const moe_config_t* c, const void* x, const void* router_w, const float* bias,
                          float* logits, int32_t* ids, float* tw, float* zw, float* scratch, hipStream_t s) {
  const bool inv = c->row_invariant != 0;
  const int slices = moe::router_slices(c->num_tokens, c->hidden, c->router_width, inv);
  float* part = slices > 1 ? scratch : logits;
  MOE_HIP(moe::launch_router_logits(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(router_w), part,
                                    c->num_tokens, c->hidden, c->router_width, slices, inv, s));
  MOE_HIP(moe::launch_topk(part, slices, logits, bias, ids, tw, zw, c->num_tokens, c->router_width, c->num_experts,
                           c->top_k, c->scoring, c->renormalize, c->routed_scale, s));
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_<unknown>";
}

const char* moe_last_error(void) { return g_err; }

moe_status_t moe_workspace_layout(const moe_config_t* cfg, moe_workspace_layout_t* layout) {
  MOE_RET(check_config(cfg));
  MOE_CHECK(layout != nullptr, MOE_ERR_INVALID, "layout is NULL");
  compute_layout(cfg, layout);
  return ok();
}

moe_status_t moe_workspace_size(const moe_config_t* cfg, size_t* bytes) {
  MOE_RET(check_config(cfg));
  MOE_CHECK(bytes != nullptr, MOE_ERR_INVALID, "bytes is NULL");
  moe_workspace_layout_t L;
  compute_layout(cfg, &L);
  *bytes = L.total;
  return ok();
}

moe_status_t moe_route_topk(const moe_config_t* cfg, const void* x, const void* router_w,
                            const float* correction_bias, float* logits, int32_t* topk_ids, float* topk_w,
                            float* zero_w, void* ws, size_t ws_bytes, void* stream) {
  MOE_RET(check_config(cfg));
  moe_workspace_layout_t L;
  compute_layout(cfg, &L);
  MOE_CHECK(ws_bytes >= L.total, MOE_ERR_WORKSPACE, "workspace too small: need %zu bytes, have %zu", L.total,
            ws_bytes);
  if (cfg->num_tokens == 0) return ok();
  MOE_RET(check_ptr(x, 16, "x"));
  MOE_RET(check_ptr(router_w, 16, "router_w"));
  if (correction_bias) MOE_RET(check_ptr(correction_bias, 4, "correction_bias"));
  MOE_RET(check_ptr(logits, 4, "logits"));
  MOE_RET(check_ptr(topk_ids, 4, "topk_ids"));
  MOE_RET(check_ptr(topk_w, 4, "topk_w"));
  if (zero_w) MOE_RET(check_ptr(zero_w, 4, "zero_w"));
  MOE_RET(check_ptr(ws, 256, "ws"));
  MOE_RET(launch_route(cfg, x, router_w, correction_bias, logits, topk_ids, topk_w, zero_w,
                       reinterpret_cast<float*>(static_cast<char*>(ws) + L.scratch), static_cast<hipStream_t>(stream)));
  return ok();
}

moe_status_t moe_permute(const moe_config_t* cfg, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
                         int32_t* sorted_ids, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
  MOE_RET(check_config(cfg));
  MOE_RET(check_ptr(counts, 4, "counts"));
  MOE_RET(check_ptr(offsets, 4, "offsets"));
  moe_workspace_layout_t L;
  compute_layout(cfg, &L);
  MOE_CHECK(ws_bytes >= L.total, MOE_ERR_WORKSPACE, "workspace too small: need %zu bytes, have %zu", L.total,
            ws_bytes);
  MOE_RET(check_ptr(ws, 256, "ws"));
  if (cfg->num_tokens > 0) {
    MOE_RET(check_ptr(topk_ids, 4, "topk_ids"));
    MOE_RET(check_ptr(sorted_ids, 4, "sorted_ids"));
    MOE_RET(check_ptr(inv_perm, 4, "inv_perm"));
  }
  const int P = cfg->num_tokens * cfg->top_k;
  int32_t* hist = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.scratch);
  MOE_HIP(moe::launch_permute(topk_ids, P, cfg->router_width, counts, offsets, sorted_ids, inv_perm, hist, nullptr,
                              static_cast<hipStream_t>(stream)));
  return ok();
}

moe_status_t moe_quantize_fp8(const moe_config_t* cfg, const void* x, uint8_t* xq, float* x_scales, void* stream) {
  MOE_RET(check_config(cfg));
  if (cfg->num_tokens == 0) return ok();
  MOE_RET(check_ptr(x, 16, "x"));
  MOE_RET(check_ptr(xq, 16, "xq"));
  MOE_RET(check_ptr(x_scales, 4, "x_scales"));
  MOE_HIP(moe::launch_quant_fp8(static_cast<const uint16_t*>(x), xq, x_scales, cfg->num_tokens, cfg->hidden,
                                static_cast<hipStream_t>(stream)));
  return ok();
}

moe_status_t moe_grouped_gemm(const moe_config_t* cfg, int32_t stage, int32_t group, const moe_weights_t* w,
                              const void* a, const float* a_scales, const int32_t* sorted_ids,
                              const int32_t* offsets, void* out, float* out_scales, void* ws, size_t ws_bytes,
                              void* stream) {
  MOE_RET(check_config(cfg));
  MOE_CHECK(stage == MOE_STAGE_GATE_UP || stage == MOE_STAGE_DOWN, MOE_ERR_INVALID,
            "stage %d is not a MOE_STAGE_* value", stage);
  MOE_CHECK(group == MOE_GROUP_ROUTED || group == MOE_GROUP_SHARED, MOE_ERR_INVALID,
            "group %d is not a MOE_GROUP_* value", group);
  MOE_CHECK(w != nullptr, MOE_ERR_INVALID, "weights is NULL");
  const bool fp8 = cfg->weight_dtype != MOE_WEIGHTS_BF16;  // scaled weights, e4m3 activations
  const bool shared = group == MOE_GROUP_SHARED;
  if (shared) MOE_CHECK(cfg->shared_inter > 0, MOE_ERR_INVALID, "MOE_GROUP_SHARED with shared_inter == 0");
  if (cfg->num_tokens == 0) return ok();
  MOE_RET(check_ptr(a, 16, "a"));
  MOE_RET(check_ptr(out, 16, "out"));
  if (fp8) {
    MOE_RET(check_ptr(a_scales, 4, "a_scales"));
    if (stage == MOE_STAGE_GATE_UP) MOE_RET(check_ptr(out_scales, 4, "out_scales"));
  }
  if (!shared) {
    MOE_RET(check_ptr(offsets, 4, "offsets"));
    if (stage == MOE_STAGE_GATE_UP) MOE_RET(check_ptr(sorted_ids, 4, "sorted_ids"));
    if (stage == MOE_STAGE_GATE_UP) {
      MOE_RET(check_ptr(w->gate_w, 8, "gate_w table"));
      MOE_RET(check_ptr(w->up_w, 8, "up_w table"));
      if (fp8) {
        MOE_RET(check_ptr(w->gate_s, 8, "gate_s table"));
        MOE_RET(check_ptr(w->up_s, 8, "up_s table"));
      }
    } else {
      MOE_RET(check_ptr(w->down_w, 8, "down_w table"));
      if (fp8) MOE_RET(check_ptr(w->down_s, 8, "down_s table"));
    }
  } else {
    if (stage == MOE_STAGE_GATE_UP) {
      MOE_RET(check_ptr(w->sh_gate_w, 16, "sh_gate_w"));
      MOE_RET(check_ptr(w->sh_up_w, 16, "sh_up_w"));
      if (fp8) {
        MOE_RET(check_ptr(w->sh_gate_s, 4, "sh_gate_s"));
        MOE_RET(check_ptr(w->sh_up_s, 4, "sh_up_s"));
      }
    } else {
      MOE_RET(check_ptr(w->sh_down_w, 16, "sh_down_w"));
      if (fp8) MOE_RET(check_ptr(w->sh_down_s, 4, "sh_down_s"));
    }
  }
  moe::GroupedGemmArgs g = gemm_args(cfg, stage, group, w, a, a_scales, sorted_ids, offsets, out, out_scales);
  if (ws != nullptr) {  // with a whole workspace: the same launch choices as moe_forward's
    moe_workspace_layout_t L;
    compute_layout(cfg, &L);
    if (ws_bytes >= L.total) {
      MOE_RET(check_ptr(ws, 256, "ws"));
      g = with_split(g, L, static_cast<char*>(ws));
    }
  }
  MOE_RET(run_gemm(cfg, g, static_cast<hipStream_t>(stream)));
  return ok();
}

moe_status_t moe_unpermute_reduce(const moe_config_t* cfg, const void* y_sorted, const int32_t* inv_perm,
                                  const int32_t* topk_ids, const float* topk_w, const void* x,
                                  const void* shared_y, const void* shared_gate, void* out, void* stream) {
  MOE_RET(check_config(cfg));
  if (cfg->num_tokens == 0) return ok();
  MOE_RET(check_ptr(y_sorted, 16, "y_sorted"));
  MOE_RET(check_ptr(inv_perm, 4, "inv_perm"));
  MOE_RET(check_ptr(topk_ids, 4, "topk_ids"));
  MOE_RET(check_ptr(topk_w, 4, "topk_w"));
  MOE_RET(check_ptr(x, 16, "x"));
  if (shared_y) MOE_RET(check_ptr(shared_y, 16, "shared_y"));
  if (shared_y && shared_gate) MOE_RET(check_ptr(shared_gate, 16, "shared_gate"));
  MOE_RET(check_ptr(out, 16, "out"));
  const moe::ReduceArgs r{inv_perm,
                          topk_ids,
                          topk_w,
                          static_cast<const uint16_t*>(x),
                          static_cast<const uint16_t*>(shared_y),
                          shared_y ? static_cast<const uint16_t*>(shared_gate) : nullptr,
                          static_cast<uint16_t*>(out),
                          cfg->num_tokens,
                          cfg->hidden,
                          cfg->top_k,
                          cfg->num_experts};
  MOE_HIP(moe::launch_unpermute_reduce(static_cast<const uint16_t*>(y_sorted), r, static_cast<hipStream_t>(stream)));
  return ok();
}

moe_status_t moe_forward(const moe_config_t* cfg, const moe_weights_t* w, const void* x, void* out, void* ws,
                         size_t ws_bytes, void* stream) {
  MOE_RET(check_config(cfg));
  MOE_RET(check_weights(cfg, w));
  moe_workspace_layout_t L;
  compute_layout(cfg, &L);
  MOE_CHECK(ws_bytes >= L.total, MOE_ERR_WORKSPACE, "workspace too small: need %zu bytes, have %zu", L.total,
            ws_bytes);
  if (cfg->num_tokens == 0) return ok();
  MOE_RET(check_ptr(x, 16, "x"));
  MOE_RET(check_ptr(out, 16, "out"));
  MOE_RET(check_ptr(ws, 256, "ws"));
  const moe_config_t& c = *cfg;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  auto at = [&](size_t off) -> void* { return off == SIZE_MAX ? nullptr : base + off; };
  float* logits = static_cast<float*>(at(L.logits));
  int32_t* ids = static_cast<int32_t*>(at(L.topk_ids));
  float* tw = static_cast<float*>(at(L.topk_w));
  float* zw = static_cast<float*>(at(L.zero_w));
  int32_t* counts = static_cast<int32_t*>(at(L.counts));
  int32_t* offsets = static_cast<int32_t*>(at(L.offsets));
  int32_t* sorted_ids = static_cast<int32_t*>(at(L.sorted_ids));
  int32_t* inv_perm = static_cast<int32_t*>(at(L.inv_perm));
  int32_t* hist = static_cast<int32_t*>(at(L.scratch));
  const int P = c.num_tokens * c.top_k;
  int32_t* sync = static_cast<int32_t*>(at(L.sync));
  int32_t* queue = nullptr;  // tile counters of the GEMMs (prefill routing only)
  // small batch: router GEMM, then top-K and the sort in one block (both in one launch for decode
  // batches), which also zeroes the counters and the error word of the one-launch decode experts path
  const bool small = moe::topk_sort_small_fits(c.num_tokens, c.top_k);
  const bool fused = small && experts_fused(cfg);
  if (small && c.row_invariant == 0 && moe::route_small_fits(c.num_tokens, c.top_k, c.router_width)) {
    // decode: router GEMV, top-K and the sort in one launch
    MOE_HIP(moe::launch_route_small(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w->router_w),
                                    logits, w->correction_bias, ids, tw, zw, counts, offsets, sorted_ids, inv_perm,
                                    sync, reinterpret_cast<unsigned long long*>(hist), fused, next_route_seq(),
                                    c.num_tokens, c.hidden, c.router_width,
                                    c.num_experts, c.top_k, c.scoring, c.renormalize, c.routed_scale, s));
  } else if (small) {
    const bool inv = c.row_invariant != 0;
    const int slices = moe::router_slices(c.num_tokens, c.hidden, c.router_width, inv);
    float* part = slices > 1 ? reinterpret_cast<float*>(hist) : logits;
    MOE_HIP(moe::launch_router_logits(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w->router_w),
                                      part, c.num_tokens, c.hidden, c.router_width, slices, inv, s));
    MOE_HIP(moe::launch_topk_sort_small(part, slices, logits, w->correction_bias, ids, tw, zw, counts, offsets,
                                        sorted_ids, inv_perm, fused ? sync : nullptr, moe::kSyncCounters, c.num_tokens,
                                        c.router_width, c.num_experts, c.top_k, c.scoring, c.renormalize,
                                        c.routed_scale, s));
  } else {
    MOE_RET(launch_route(cfg, x, w->router_w, w->correction_bias, logits, ids, tw, zw, reinterpret_cast<float*>(hist),
                         s));
    // the sort also zeroes the GEMMs' tile counters, which each launch that takes them leaves zero
    queue = sync + moe::kSyncQueue;
    MOE_HIP(moe::launch_permute(ids, P, c.router_width, counts, offsets, sorted_ids, inv_perm, hist, queue, s));
  }
  return run_experts(cfg, w, x, ids, tw, offsets, sorted_ids, inv_perm, out, L, base, fused, queue, s);
}

moe_status_t moe_experts_forward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                                 const int32_t* topk_ids, const float* topk_w, const int32_t* offsets,
                                 const int32_t* sorted_ids, const int32_t* inv_perm, void* out, void* ws,
                                 size_t ws_bytes, void* stream) {
  MOE_RET(check_config(cfg));
  MOE_RET(check_weights(cfg, w));
  moe_workspace_layout_t L;
  compute_layout(cfg, &L);
  MOE_CHECK(ws_bytes >= L.total, MOE_ERR_WORKSPACE, "workspace too small: need %zu bytes, have %zu", L.total,
            ws_bytes);
  if (cfg->num_tokens == 0) return ok();
  MOE_RET(check_ptr(x, 16, "x"));
  MOE_RET(check_ptr(topk_ids, 4, "topk_ids"));
  MOE_RET(check_ptr(topk_w, 4, "topk_w"));
  MOE_RET(check_ptr(offsets, 4, "offsets"));
  MOE_RET(check_ptr(sorted_ids, 4, "sorted_ids"));
  MOE_RET(check_ptr(inv_perm, 4, "inv_perm"));
  MOE_RET(check_ptr(out, 16, "out"));
  MOE_RET(check_ptr(ws, 256, "ws"));
  return run_experts(cfg, w, x, topk_ids, topk_w, offsets, sorted_ids, inv_perm, out, L, static_cast<char*>(ws),
                     experts_fused(cfg), nullptr, static_cast<hipStream_t>(stream));
}

moe_status_t moe_forward_noalloc(const moe_config_t* cfg, const moe_weights_t* w, const void* x, void* out,
                                 void* stream) {
  MOE_RET(check_config(cfg));
  moe_workspace_layout_t L;
  compute_layout(cfg, &L);
  MOE_CHECK(L.total <= (size_t)MOE_NOALLOC_WORKSPACE_BYTES, MOE_ERR_WORKSPACE,
            "moe_forward_noalloc: this layer needs %zu bytes of workspace, more than the static %zu bytes; "
            "call moe_forward with a workspace of its own",
            L.total, (size_t)MOE_NOALLOC_WORKSPACE_BYTES);
  if (cfg->num_tokens == 0) return ok();
  void* ws = nullptr;
  MOE_RET(scratch_on_current_device(&ws));
  return moe_forward(cfg, w, x, out, ws, (size_t)MOE_NOALLOC_WORKSPACE_BYTES, stream);
}

}  // extern "C"
