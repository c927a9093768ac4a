/*
 * libmoe: the mixture-of-experts layer forward on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every tensor argument is a DEVICE pointer to memory the caller owns;
 * only the two structs (moe_config_t, moe_weights_t) and the size_t* out-arg of
 * moe_workspace_size live in host memory.  The library never allocates, frees,
 * synchronises or copies to the host: every call only enqueues kernels on
 * `stream` (a hipStream_t; NULL is the null stream), so a sequence of calls can
 * be captured into a HIP graph.  The caller keeps every buffer alive until the
 * stream has finished the work.
 *
 * Layouts are row-major.  "bf16" is bfloat16 (uint16 bit patterns), "e4m3" is
 * the OCP FP8 E4M3 format (bias 7, max 448, no infinities).  Weights follow the
 * [out, in] convention of a linear layer: W_gate, W_up are [I, H], W_down is
 * [H, I].  Ids are int32.  N = num_tokens, K = top_k, R = router_width,
 * E = num_experts (real experts; router columns [E, R) are zero-computation
 * "identity" experts), I = inter, Is = shared_inter, P = N*K.
 *
 * Errors: every call validates its arguments before it launches anything and
 * returns a status; moe_last_error() returns a message for the calling thread's
 * last failure.  No call falls back to another method silently.
 *
 * The method follows five pages of MoE dispatch code from two inference
 * engines; the citations below name the page (its source file path) and the
 * function or comment on it.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,     /* null/misaligned pointer, inconsistent sizes, bad enum value */
  MOE_ERR_UNSUPPORTED = 2, /* a valid request this build does not implement (named in the message) */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than moe_workspace_size() ("need X bytes, have Y") */
  MOE_ERR_HIP = 4          /* a HIP runtime error from a launch */
} moe_status_t;

enum { MOE_SCORING_SOFTMAX = 0, MOE_SCORING_SIGMOID = 1, MOE_SCORING_SQRTSOFTPLUS = 2 };
enum { MOE_WEIGHTS_BF16 = 0, MOE_WEIGHTS_FP8_E4M3 = 1, MOE_WEIGHTS_MXFP4 = 2 };
enum { MOE_STAGE_GATE_UP = 0, MOE_STAGE_DOWN = 1 };
enum { MOE_GROUP_ROUTED = 0, MOE_GROUP_SHARED = 1 };

/* Layer hyper-parameters (the model-config fields the pages read: hidden_size,
 * num_experts, num_experts_per_tok, moe_intermediate_size,
 * shared_expert_intermediate_size, scoring_func, norm_topk_prob,
 * routed_scaling_factor, and the router width router_logits_n).
 * Supported: N >= 0; H and I multiples of 128; Is = 0 or a multiple of 128;
 * 1 <= E <= R <= 1024; 1 <= K <= min(R, 32). */
typedef struct {
  int32_t num_tokens;   /* N */
  int32_t hidden;       /* H */
  int32_t num_experts;  /* E */
  int32_t router_width; /* R */
  int32_t top_k;        /* K */
  int32_t inter;        /* I */
  int32_t shared_inter; /* Is; 0 = no shared expert */
  int32_t scoring;      /* MOE_SCORING_* */
  int32_t renormalize;  /* nonzero: divide the K weights by their sum */
  float routed_scale;   /* multiplies the (renormalised) weights */
  int32_t weight_dtype; /* MOE_WEIGHTS_*: type of the expert (routed and shared) weights */
  int32_t row_invariant; /* 0 or 1.  1: every token's output bits are independent of the batch it
                            comes in (forward_prefill.rs page, prefill_row_invariant: a prompt's rows
                            get the same bits in a cold pass and in a short replay of its tail).  The
                            same kernels and sum orders then run at every N (the router split fixed by
                            H, the general grouped GEMMs, the separate reduce), at the cost of the
                            decode-shaped kernels' speed.  0: the fastest kernels for each N. */
} moe_config_t;

/* Weights of one layer.  The router is always bf16.  Routed experts are reached
 * through DEVICE arrays of E device pointers (per-expert pointer tables, as the
 * pages keep them), so experts may live anywhere in device memory.
 * bf16: gate_w[e], up_w[e] -> [I, H] bf16; down_w[e] -> [H, I] bf16.
 * fp8:  the same matrices as e4m3 codes, plus one fp32 scale per 128x128 block:
 *       gate_s[e], up_s[e] -> [I/128, H/128]; down_s[e] -> [H/128, I/128]
 *       (dequantised weight = code * scale of its block).
 * mxfp4 (OCP Microscaling MXFP4; the forward.rs page's MXFP4 / E8M0 expert arm):
 *       each matrix [rows, K] as packed FP4 E2M1 codes [rows, K/2] uint8 (column 2j in
 *       the low nibble of byte j) plus one E8M0 code per row and 32 columns,
 *       [rows, K/32] uint8, passed in the *_s pointers (4-byte aligned); dequantised
 *       weight = e2m1(code) * 2^(e8m0 - 127).  Activations and h are e4m3 with fp32
 *       per-128 scales as on the fp8 path.
 * The shared expert, if Is > 0, is given directly (not through tables) with
 * Is in place of I.  Pointers must be 16-byte aligned. */
typedef struct {
  const void* router_w;        /* [R, H] bf16 */
  const float* correction_bias; /* [R] fp32, or NULL (no bias) */
  const void* const* gate_w;   /* device array [E] */
  const void* const* up_w;     /* device array [E] */
  const void* const* down_w;   /* device array [E] */
  const float* const* gate_s;  /* device array [E]; fp8 only, else NULL */
  const float* const* up_s;
  const float* const* down_s;
  const void* sh_gate_w; /* [Is, H]; NULL when Is == 0 */
  const void* sh_up_w;   /* [Is, H] */
  const void* sh_down_w; /* [H, Is] */
  const float* sh_gate_s; /* fp8 only: [Is/128, H/128] */
  const float* sh_up_s;
  const float* sh_down_s; /* [H/128, Is/128] */
  const void* sh_expert_gate; /* [H] bf16: the shared expert's sigmoid gate row, or NULL (weight 1);
                                 must be NULL when Is == 0 */
} moe_weights_t;

/* Bytes of device workspace that moe_forward, moe_experts_forward and moe_permute need for `cfg`
 * (a function of the sizes only; 256-byte aligned pieces). */
moe_status_t moe_workspace_size(const moe_config_t* cfg, size_t* bytes);

/* Router gate GEMM + scoring + top-K selection.  ws: at least
 * moe_workspace_size(cfg) bytes (split-K partial logits are staged there).
 * forward_prefill.rs page, MoeLayer::forward_prefill gate GEMM and top-K steps;
 * forward.rs page, MoeLayer::forward top-K arms (moe_topk_softmax;
 * moe_topk_sigmoid with the correction bias used for selection only;
 * moe_topk_softmax_bias with the zero-expert fold into zero_accum;
 * moe_topk_sqrtsoftplus, the DeepSeek-V4 arm: scores = sqrtsoftplus(logits)).
 *   logits[t,r] = sum_h x[t,h] * router_w[r,h]          (fp32 accumulation)
 *   p = softmax over all R columns, sigmoid, or sqrt(softplus) with
 *       softplus(z) = ln(1 + e^z)                          (fp32)
 *   ids[t,0..K) = the K largest p + bias (bias 0 if NULL), slots in descending
 *                 order, exact ties to the lower column
 *   w[t,k] = p[ids] (unbiased); / sum_k when renormalize; * routed_scale
 *   zero_w[t] = sum of w[t,k] over slots with ids >= E
 * x [N, H] bf16; router_w [R, H] bf16; correction_bias [R] fp32 or NULL;
 * logits [N, R] fp32 (required: the scores are staged there); topk_ids [N, K]
 * int32; topk_w [N, K] fp32; zero_w [N] fp32 or NULL. */
moe_status_t moe_route_topk(const moe_config_t* cfg, const void* x, const void* router_w,
                            const float* correction_bias, float* logits, int32_t* topk_ids, float* topk_w,
                            float* zero_w, void* ws, size_t ws_bytes, void* stream);

/* Count and sort the expanded (token, slot) rows by expert.
 * forward_prefill.rs page, moe_sort_by_expert (sorted_token_ids, expert_offsets,
 * token_to_perm).  Every router column has a bucket; identity experts sort to
 * the tail.  Stable: within a bucket rows keep ascending expanded index t*K+k.
 *   counts[r] = #{(t,k): ids[t,k] == r}                  [R]
 *   offsets   = exclusive prefix sum of counts            [R + 1], offsets[R] = P
 *   sorted_ids[p] = the expanded index t*K+k at sorted position p   [P]
 *   inv_perm[t*K+k] = its sorted position p (token_to_perm)          [P]
 * The ids are device data the host cannot check: an id outside [0, R) is not
 * counted and its row is not written, so the outputs are then not a
 * permutation (ids from moe_route_topk are always in range).
 * ws: at least moe_workspace_size(cfg) bytes. */
moe_status_t moe_permute(const moe_config_t* cfg, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
                         int32_t* sorted_ids, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);

/* fp8 activation quantisation (the FP8 expert path: activations quantised per
 * token and per 128-column group).  For each row and each group of 128 columns:
 *   amax = max |x|; inv = 448 / amax (correctly rounded fp32);
 *   xq = e4m3(x * inv) (round to nearest even, saturating); x_scales = amax / 448;
 *   an all-zero group gets x_scales = 1 and zero codes.
 * x [N, H] bf16 -> xq [N, H] e4m3 codes, x_scales [N, H/128] fp32. */
moe_status_t moe_quantize_fp8(const moe_config_t* cfg, const void* x, uint8_t* xq, float* x_scales,
                              void* stream);

/* Grouped expert GEMM over the rows sorted by expert.
 * forward_prefill.rs page, run_routed_grouped_gemm (grouped gate/up GEMM,
 * activation, grouped down GEMM over expert_offsets / sorted_token_ids) and the
 * shared expert (run_shared_expert_prefill).
 * stage MOE_STAGE_GATE_UP:  out[p, :] = silu(a_p W_gate^T) * (a_p W_up^T)     [rows, I]
 * stage MOE_STAGE_DOWN:     out[p, :] = a_p W_down^T                            [rows, H]
 * group MOE_GROUP_ROUTED: rows p in [offsets[e], offsets[e+1]) use expert e's
 *   weights, for e < E (identity-expert rows at the tail are not computed and
 *   not written).  GATE_UP reads a_p = a[sorted_ids[p] / K] (a is [N, H], the
 *   token's row); DOWN reads a_p = a[p] (a is the GATE_UP output, [P, I]).
 * group MOE_GROUP_SHARED: rows t in [0, N) use the shared expert (Is in place
 *   of I); a_t = a[t]; sorted_ids and offsets are ignored (may be NULL).
 * bf16 weights: a and out are bf16; a_scales and out_scales are ignored.
 * fp8 and mxfp4 weights: a is e4m3 with a_scales [rows of a, cols/128] fp32 (from
 *   moe_quantize_fp8 for GATE_UP, from the GATE_UP output for DOWN); GATE_UP
 *   writes e4m3 codes + out_scales [P or N, I/128] quantised per 128 columns
 *   like moe_quantize_fp8; DOWN writes bf16.
 * ws: NULL, or at least moe_workspace_size(cfg) bytes (256-byte aligned, any contents).  With
 *   a workspace, a routed bf16 launch makes moe_forward's choices: for layers that have the `split`
 *   piece (moe_workspace_layout), when the last round of tiles fills at most half of the GPU its tiles
 *   are split along K into parts whose fp32 sums are added in part order by the last part to arrive.
 *   Without one it never splits, and a split tile's outputs can then differ from moe_forward's in
 *   their last bits (a different order of the same sums).  Calls that overlap on one workspace race. */
moe_status_t moe_grouped_gemm(const moe_config_t* cfg, int32_t stage, int32_t group, const moe_weights_t* w,
                              const void* a, const float* a_scales, const int32_t* sorted_ids,
                              const int32_t* offsets, void* out, float* out_scales, void* ws, size_t ws_bytes,
                              void* stream);

/* Unpermute with the top-K-weighted reduce, plus the shared-expert and
 * zero-computation-expert blends, rounded once to bf16.
 * forward_prefill.rs page, moe_unpermute_reduce_indexed and the shared blend
 * (output += sigmoid(input . shared_expert_gate) * shared, weight 1 without a
 * shared_expert_gate); forward.rs page, MoeLayer::apply_zero_expert
 * (out[t,:] += zero_accum[t] * x[t,:]).
 *   g[t] = sigmoid(sum_h x[t,h] * shared_gate[h])  (fp32), or 1 if shared_gate is NULL
 *   out[t,:] = bf16( sum_{k: ids<E} w[t,k] * y_sorted[inv_perm[t*K+k], :]
 *                    + (sum_{k: ids>=E} w[t,k]) * x[t,:] + g[t] * shared_y[t,:] )   (fp32 sum)
 * y_sorted [P, H] bf16 (the DOWN output); inv_perm [P]; topk_ids, topk_w [N, K];
 * x [N, H] bf16; shared_y [N, H] bf16 or NULL; shared_gate [H] bf16 or NULL (ignored
 * without shared_y); out [N, H] bf16. */
moe_status_t moe_unpermute_reduce(const moe_config_t* cfg, const void* y_sorted, const int32_t* inv_perm,
                                  const int32_t* topk_ids, const float* topk_w, const void* x,
                                  const void* shared_y, const void* shared_gate, void* out, void* stream);

/* The whole layer: route -> sort -> [quantise] -> gate/up (+ shared) -> down
 * (+ shared) -> unpermute-reduce, on one stream with no host synchronisation.
 * Same result as composing the calls above.  forward_prefill.rs page,
 * MoeLayer::forward_prefill (the grouped data flow); forward.rs page,
 * MoeLayer::forward and apply_zero_expert.
 * x [N, H] bf16 -> out [N, H] bf16; ws: at least moe_workspace_size(cfg) bytes,
 * with any contents (a decode batch's routing launch hands its logits over in
 * the `scratch` piece as words tagged with a value of that very launch, and
 * counts a word only when it carries that value).  Calls that overlap on one
 * workspace race. */
moe_status_t moe_forward(const moe_config_t* cfg, const moe_weights_t* w, const void* x, void* out, void* ws,
                         size_t ws_bytes, void* stream);

/* The expert half of the layer for a routing computed elsewhere (moe_route_topk
 * and moe_permute, or moe_forward's own): [quantise] -> gate/up (+ shared) ->
 * down (+ shared) -> unpermute-reduce with the blends.  Same result as
 * composing moe_quantize_fp8, moe_grouped_gemm and moe_unpermute_reduce.
 * forward_prefill.rs page, run_routed_grouped_gemm, run_shared_expert_prefill
 * and moe_unpermute_reduce_indexed; forward.rs page, apply_zero_expert.
 * x [N, H] bf16; topk_ids, topk_w [N, K]; offsets [R + 1], sorted_ids [P],
 * inv_perm [P] as moe_permute writes them; out [N, H] bf16.
 * ws: at least moe_workspace_size(cfg) bytes.  With bf16 weights, H <= 65536 and
 * a few rows per touched expert (decode) the routed GEMMs and the reduce run as
 * one launch whose tiles wait on counters in the workspace's `sync` piece.  That
 * piece is the first 8232 bytes of every workspace, whatever the sizes, and its
 * counters must hold zeros when the call starts: zero them once (e.g. zero the
 * whole workspace after allocating it); every call of this library leaves them
 * zero, so the workspace can then serve any batch size and layer shape.
 * The int32 at byte offset `sync_error` (moe_workspace_layout) is set to 1 if a
 * tile's bounded wait for another tile ever expires (an error of this library,
 * not of the input); the output of that call is then undefined.  No launch
 * clears the word: moe_forward clears it when it starts, and otherwise the
 * caller does.  Calls that overlap on one workspace race. */
moe_status_t moe_experts_forward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                                 const int32_t* topk_ids, const float* topk_w, const int32_t* offsets,
                                 const int32_t* sorted_ids, const int32_t* inv_perm, void* out, void* ws,
                                 size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and result, with the workspace taken from a static array of
 * MOE_NOALLOC_WORKSPACE_BYTES inside the library instead of from the caller.
 * Each GPU the library runs on holds its own copy of that array from the
 * library's load until the process ends; the call uses the copy of the current
 * device (`stream` must belong to it).  Nothing is allocated or freed.
 * A layer whose moe_workspace_size exceeds MOE_NOALLOC_WORKSPACE_BYTES is
 * refused with MOE_ERR_WORKSPACE before anything is launched (32 MiB serves,
 * e.g., decode batches up to a few hundred tokens at H 2048, 128 experts, top-8).
 * Every call on one GPU shares that GPU's array and leaves its contents there
 * (the next call accepts any contents): calls that overlap on one GPU, from
 * several streams or threads, race and give undefined results.
 * x [N, H] bf16 -> out [N, H] bf16. */
#define MOE_NOALLOC_WORKSPACE_BYTES (32u << 20)
moe_status_t moe_forward_noalloc(const moe_config_t* cfg, const moe_weights_t* w, const void* x, void* out,
                                 void* stream);

/* Offsets of the intermediates inside the moe_forward workspace, so a caller
 * can inspect them after moe_forward (all in bytes from the workspace start;
 * a piece that the config does not use has offset SIZE_MAX).  `sync` (always 0)
 * holds the counters of the one-launch decode experts path and `sync_error` its
 * error word (see moe_experts_forward), the arrival counters of split tiles, and
 * the per-XCD tile counters that moe_forward's sort zeroes for the GEMMs after it.
 * `split` holds the parts' fp32 partial sums of split tiles: present for bf16
 * layers of at least 2048 routed rows with H or I of at least 4096, without a
 * shared expert and not row-invariant (see moe_grouped_gemm). */
typedef struct {
  size_t logits, topk_ids, topk_w, zero_w, counts, offsets, sorted_ids, inv_perm;
  size_t xq, x_scales, h, h_scales, y, shared_h, shared_h_scales, shared_y, scratch, sync, sync_error, split, total;
} moe_workspace_layout_t;
moe_status_t moe_workspace_layout(const moe_config_t* cfg, moe_workspace_layout_t* layout);

const char* moe_status_str(moe_status_t status);
const char* moe_last_error(void); /* thread-local; "" when the last call succeeded */

#ifdef __cplusplus
}
#endif
#endif
