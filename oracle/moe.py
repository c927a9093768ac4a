"""The MoE layer forward, written out plainly in float64 on the CPU.

TEST INFRASTRUCTURE ONLY.  See ``oracle/__init__.py``.

Sources (five web pages of host-side MoE dispatch code from two inference
engines; no page prints kernel source or numbers for this path):

* "metrale_model_layers/layers/moe/forward_prefill.rs", doc comment of
  ``MoeLayer::forward_prefill`` and its steps: gate GEMM, top-K, sort by
  expert (``moe_sort_by_expert`` and its four outputs), grouped gate/up GEMM,
  activation, grouped down GEMM, ``moe_unpermute_reduce_indexed`` and the
  shared-expert blend: output += sigmoid(input . shared_expert_gate) * shared,
  weight 1 when the layer has no shared_expert_gate.
* "spark_model/layers/moe/forward.rs", ``MoeLayer::forward``: the top-K
  scoring arms (softmax; sigmoid + correction bias for selection with
  unbiased, renormalised, scaled weights; softmax + correction bias with the
  zero-computation experts folded into ``zero_accum``; the DeepSeek-V4
  sqrtsoftplus + correction bias arm: scores = sqrtsoftplus(gate_logits),
  indices = topk(scores + bias), weights = scores[indices] / their sum) and the
  doc comment of ``MoeLayer::apply_zero_expert`` (out[t,:] += zero_accum[t] *
  x[t,:]).
* "spark_model/layers/moe/forward_batched.rs", ``MoeLayer::forward_batched``:
  the router width R differs from the expert count E only when the router also
  scores the zero-computation experts.

Readings of points the pages leave open (each is also listed with the design
notes): logits and scores in float64 (the GPU uses fp32; never bf16); ties in
the selection score go to the lower router column, slots ordered by
descending selection score; the sort is stable in the expanded index t*K+k and
``sorted_token_ids`` stores that expanded index; h = silu(g)*u is rounded to
the expert GEMM operand type (bf16, or e4m3 with per-128 scales) before the
down projection, nothing else is rounded until the one final bf16 rounding;
sqrtsoftplus(z) is sqrt(softplus(z)) = sqrt(ln(1 + e^z)) (the pages only name
it); the shared-expert gate is one bf16 weight row [H] and its dot product with
the token's bf16 input is exact in float64.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional

import numpy as np

from .codecs import bf16_to_f64, e4m3_decode, e4m3_encode, f64_to_bf16, mxfp4_dequant

FP8_BLOCK = 128
E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    """The layer's hyper-parameters, as named by the pages' model config."""

    hidden: int  # hidden_size (H)
    num_experts: int  # num_experts (E), real SwiGLU experts
    router_width: int  # router_logits_n (R); columns [E, R) are identity experts
    top_k: int  # num_experts_per_tok (K)
    inter: int  # moe_intermediate_size (I)
    shared_inter: int  # shared_expert_intermediate_size (0: none)
    scoring: str  # scoring_func: "softmax" | "sigmoid" | "sqrtsoftplus"
    renormalize: bool  # norm_topk_prob
    routed_scale: float  # routed_scaling_factor
    weight_dtype: str  # "bf16" | "fp8" | "mxfp4" (fp8 and mxfp4 experts take fp8 activations)


# ----------------------------------------------------------------------------- routing

def router_logits(x_bits: np.ndarray, router_bits: np.ndarray) -> np.ndarray:
    """gate_logits[t, r] = sum_h x[t,h] * W_router[r,h], for every router column.

    forward_prefill.rs page, gate GEMM step; forward_batched.rs page: the router
    also scores the zero-computation experts, so r runs over the router width.
    bf16 x bf16 products are exact in float64; the sum is float64.
    """
    return bf16_to_f64(x_bits) @ bf16_to_f64(router_bits).T


def scores(logits: np.ndarray, scoring: str) -> np.ndarray:
    """Router scores: softmax over all R columns, the logistic sigmoid, or
    sqrt(softplus).

    forward.rs page, ``MoeLayer::forward`` top-K arms (``moe_topk_softmax``;
    the sigmoid + correction bias comment: scores = sigmoid(gate_logits); the
    DeepSeek-V4 comment: scores = sqrtsoftplus(gate_logits)).  softplus(z) =
    ln(1 + e^z), written as max(z, 0) + ln(1 + e^-|z|) so that no exponential
    overflows.
    """
    if scoring == "softmax":
        z = logits - logits.max(axis=1, keepdims=True)
        e = np.exp(z)
        return e / e.sum(axis=1, keepdims=True)
    if scoring == "sigmoid":
        return 1.0 / (1.0 + np.exp(-logits))
    if scoring == "sqrtsoftplus":
        return np.sqrt(np.maximum(logits, 0.0) + np.log1p(np.exp(-np.abs(logits))))
    raise ValueError(f"unknown scoring {scoring!r}")


def select_topk(p: np.ndarray, bias: Optional[np.ndarray], k: int):
    """indices = topk(scores + bias): the K largest selection scores per row.

    forward.rs page, sigmoid + correction bias comment (the bias steers
    SELECTION only).  Slots are ordered by descending selection score; exact
    ties go to the lower column (a stable sort of the negated scores).
    Returns (ids [N,K] int32, gap [N]) where gap is the K-th minus the
    (K+1)-th selection score (inf when K == R).
    """
    s = p if bias is None else p + bias.astype(np.float64)[None, :]
    order = np.argsort(-s, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    rows = np.arange(s.shape[0])
    if k < s.shape[1]:
        gap = s[rows, order[:, k - 1]] - s[rows, order[:, k]]
    else:
        gap = np.full(s.shape[0], np.inf)
    return ids, gap


def routing_weights(p: np.ndarray, ids: np.ndarray, renormalize: bool, routed_scale: float, num_experts: int):
    """weights = scores[indices] (unbiased), / their sum when norm_topk_prob,
    then * routed_scaling_factor; zero_accum[t] = sum of the weights of the
    selected identity experts (ids >= E).

    forward.rs page: sigmoid + correction bias comment (weights =
    scores[indices] / sum(scores[indices]), the divide toggled by
    norm_topk_prob, then the scaling factor); softmax + correction bias arm
    (unbiased softmax * scaling, zero-expert fold into zero_accum).
    """
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    w = w * routed_scale
    zero_accum = np.where(ids >= num_experts, w, 0.0).sum(axis=1)
    return w, zero_accum


# ----------------------------------------------------------------------------- sort by expert

def sort_by_expert(ids: np.ndarray, router_width: int):
    """Counting sort of the expanded (token, slot) rows by expert.

    forward_prefill.rs page, ``moe_sort_by_expert``: outputs sorted_token_ids
    [N*K], expert_offsets [E+1] and token_to_perm [N*K].  Readings: every
    router column gets a bucket (identity experts sort to the tail and are
    never computed); within a bucket rows keep ascending expanded index
    t*K+k; sorted_token_ids holds that expanded index; token_to_perm is the
    inverse permutation.
    """
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.zeros(router_width, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(router_width + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    cursor = offsets[:-1].copy()
    sorted_token_ids = np.empty(len(flat), dtype=np.int64)
    for i, e in enumerate(flat):  # ascending i keeps each bucket stable
        sorted_token_ids[cursor[e]] = i
        cursor[e] += 1
    token_to_perm = np.empty(len(flat), dtype=np.int64)
    token_to_perm[sorted_token_ids] = np.arange(len(flat))
    return (counts.astype(np.int32), offsets.astype(np.int32), sorted_token_ids.astype(np.int32),
            token_to_perm.astype(np.int32))


# ----------------------------------------------------------------------------- fp8 activations

def quantize_fp8_groups(v: np.ndarray):
    """Per row, per 128-column group: s = amax/448, code = e4m3(v * (448/amax)).

    Quantisation recipe of the FP8 workload (activations in fp8 with per-token,
    per-128 group scales).  Reading: the decision is taken in fp32, the GPU
    kernel's precision: amax of the fp32 values, inv = fp32(448/amax),
    code = e4m3_rne_satfinite(fp32(v*inv)), s = fp32(amax/448); an all-zero
    group gets s = 1 and zero codes.  Returns (codes uint8 [rows, cols],
    scales float32 [rows, cols/128]).
    """
    v = np.asarray(v, dtype=np.float32)
    rows, cols = v.shape
    assert cols % FP8_BLOCK == 0
    g = v.reshape(rows, cols // FP8_BLOCK, FP8_BLOCK)
    amax = np.abs(g).max(axis=2)
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = np.where(amax > 0, np.float32(E4M3_MAX) / safe, np.float32(1.0)).astype(np.float32)
    scaled = (g * inv[:, :, None]).astype(np.float32)
    codes = e4m3_encode(scaled).reshape(rows, cols)
    s = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0)).astype(np.float32)
    return codes, s


def dequant_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes [rows, cols] with per-row, per-128-column scales -> float64 (exact)."""
    return e4m3_decode(codes) * np.repeat(scales.astype(np.float64), FP8_BLOCK, axis=1)


def dequant_blocks(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """A weight matrix -> float64 (exact).  e4m3 codes with one fp32 scale per 128x128 block,
    or MXFP4 (packed E2M1 codes with one E8M0 scale per row and 32 columns; the scales are
    uint8 then)."""
    if scales.dtype == np.uint8:
        return mxfp4_dequant(codes, scales)
    s = np.repeat(np.repeat(scales.astype(np.float64), FP8_BLOCK, axis=0), FP8_BLOCK, axis=1)
    return e4m3_decode(codes) * s[: codes.shape[0], : codes.shape[1]]


# ----------------------------------------------------------------------------- experts

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) (no clamp)."""
    return z / (1.0 + np.exp(-z))


def gate_up_bf16(xrows: np.ndarray, wg_bits, wu_bits) -> np.ndarray:
    """h = bf16(silu(W_gate x) * (W_up x)) for each row of xrows (float64 inputs).

    forward_prefill.rs page: grouped gate/up GEMM and the activation;
    W_gate and W_up are [I, H] (out x in).  h is rounded to bf16, the down
    GEMM's operand type.  Returns bf16 bits [rows, I].
    """
    g = xrows @ bf16_to_f64(wg_bits).T
    u = xrows @ bf16_to_f64(wu_bits).T
    return f64_to_bf16(silu(g) * u)


def down_bf16(h_bits: np.ndarray, wd_bits) -> np.ndarray:
    """y = W_down h (float64, not rounded); W_down is [H, I].  forward_prefill.rs
    page: grouped down GEMM."""
    return bf16_to_f64(h_bits) @ bf16_to_f64(wd_bits).T


def swiglu_expert_bf16(xrows: np.ndarray, wg_bits, wu_bits, wd_bits) -> np.ndarray:
    """y = W_down * bf16(silu(W_gate x) * (W_up x)) for each row of xrows (float64)."""
    return down_bf16(gate_up_bf16(xrows, wg_bits, wu_bits), wd_bits)


def gate_up_fp8(xq_rows: np.ndarray, xs_rows: np.ndarray, wg, wu):
    """The gate/up GEMM and activation on e4m3 operands with fp32 block scales.

    x rows arrive quantised per 128 columns; each weight is (codes, scales per
    128x128 block).  Dequantising both operands is exact in float64, so the
    float64 product equals the sum over 128-blocks of (s_x * S_w) times the
    block's code dot product.  h is then quantised per 128 columns like x (its
    quantisation decision taken on fp32(h)).  Returns (codes, scales).
    """
    x = dequant_rows(xq_rows, xs_rows)
    g = x @ dequant_blocks(*wg).T
    u = x @ dequant_blocks(*wu).T
    return quantize_fp8_groups((silu(g) * u).astype(np.float32))


def down_fp8(hq: np.ndarray, hs: np.ndarray, wd) -> np.ndarray:
    """y = W_down h on e4m3 operands (float64 result, not rounded)."""
    return dequant_rows(hq, hs) @ dequant_blocks(*wd).T


def swiglu_expert_fp8(xq_rows: np.ndarray, xs_rows: np.ndarray, wg, wu, wd) -> np.ndarray:
    """The fp8 expert: gate_up_fp8 then down_fp8."""
    return down_fp8(*gate_up_fp8(xq_rows, xs_rows, wg, wu), wd)


# ----------------------------------------------------------------------------- the layer

@dataclasses.dataclass
class OracleResult:
    tokens: np.ndarray  # which tokens these rows are
    logits: np.ndarray  # [n, R] float64
    probs: np.ndarray  # [n, R] float64
    ids: np.ndarray  # [n, K] int32
    gap: np.ndarray  # [n] K-th minus (K+1)-th selection score
    weights: np.ndarray  # [n, K] float64
    zero_accum: np.ndarray  # [n] float64
    routed: np.ndarray  # [n, H] float64: sum_k w * y over real experts
    shared: Optional[np.ndarray]  # [n, H] float64, the shared expert's output before its gate
    shared_weight: np.ndarray  # [n] float64: sigmoid(x . shared_expert_gate), or 1
    out_f64: np.ndarray  # [n, H] float64 before the final rounding
    out_bits: np.ndarray  # [n, H] bf16 bits


ExpertFn = Callable[[int], tuple]


def shared_gate(x_bits: np.ndarray, gate_bits: Optional[np.ndarray]) -> np.ndarray:
    """Per-token weight of the shared expert: sigmoid(x[t] . shared_expert_gate),
    or 1 when the layer has no shared_expert_gate.

    forward_prefill.rs page, the shared-expert blend comment.  gate_bits is the
    gate's one weight row [H] (bf16); the dot product is float64.
    """
    if gate_bits is None:
        return np.ones(x_bits.shape[0])
    z = bf16_to_f64(x_bits) @ bf16_to_f64(gate_bits)
    return 1.0 / (1.0 + np.exp(-z))


def moe_forward(cfg: MoeConfig, x_bits: np.ndarray, router_bits: np.ndarray, bias: Optional[np.ndarray],
                expert: ExpertFn, shared: Optional[tuple], tokens: Optional[np.ndarray] = None,
                shared_gate_bits: Optional[np.ndarray] = None,
                forced_ids: Optional[np.ndarray] = None) -> OracleResult:
    """out[t] = bf16( sum_{k: id<E} w[t,k] * y_{t,k} + zero_accum[t] * x[t] + g[t] * shared[t] ),
    with g[t] = sigmoid(x[t] . shared_expert_gate), or 1 without that gate.

    Every token is independent, so ``x_bits`` may hold any subset of the
    layer's rows (``tokens`` names them, for bookkeeping only).
    ``expert(e)`` returns routed expert e's weights (bf16 bit arrays
    (Wg, Wu, Wd), or fp8 ((codes, scales) x 3)), fetched only for experts some
    row selects; ``shared`` is the shared expert in the same form or None,
    ``shared_gate_bits`` its gate row [H] (bf16 bits) or None.

    Steps as on the forward_prefill.rs page: gate GEMM, top-K, grouped
    gate/up + SwiGLU, grouped down, unpermute + top-K-weighted reduce, shared
    blend (sigmoid-gated, or weight 1); then the zero-computation experts' term of
    ``MoeLayer::apply_zero_expert`` (forward.rs page).  Reading: the three
    terms are summed in float64 and rounded to bf16 once.

    ``forced_ids`` ([n, K], optional) replaces the selected expert ids, for rows
    whose K-th and (K+1)-th selection scores are a near-tie, where a selection in
    lower precision may pick the other expert; the weights are still the unbiased
    scores of those ids, renormalised and scaled as usual (``gap`` stays the
    float64 selection's).
    """
    n = x_bits.shape[0]
    tokens = np.arange(n) if tokens is None else np.asarray(tokens)
    E, K = cfg.num_experts, cfg.top_k
    logits = router_logits(x_bits, router_bits)
    p = scores(logits, cfg.scoring)
    ids, gap = select_topk(p, bias, K)
    if forced_ids is not None:
        ids = np.asarray(forced_ids, dtype=np.int32).reshape(n, K)
    w, zero_accum = routing_weights(p, ids, cfg.renormalize, cfg.routed_scale, E)

    x64 = bf16_to_f64(x_bits)
    if cfg.weight_dtype != "bf16":  # fp8 and mxfp4 experts: e4m3 activations, per-128 scales
        xq, xs = quantize_fp8_groups(x64.astype(np.float32))
    routed = np.zeros((n, cfg.hidden), dtype=np.float64)
    for e in np.unique(ids[ids < E]):  # expert-major: fetch each touched expert once
        rows, slots = np.nonzero(ids == e)
        we = expert(int(e))
        if cfg.weight_dtype == "bf16":
            y = swiglu_expert_bf16(x64[rows], *we)
        else:
            y = swiglu_expert_fp8(xq[rows], xs[rows], *we)
        np.add.at(routed, rows, w[rows, slots][:, None] * y)

    sh = None
    if shared is not None:
        if cfg.weight_dtype == "bf16":
            sh = swiglu_expert_bf16(x64, *shared)
        else:
            sh = swiglu_expert_fp8(xq, xs, *shared)

    g = shared_gate(x_bits, shared_gate_bits)
    total = routed + zero_accum[:, None] * x64
    if sh is not None:
        total = total + g[:, None] * sh
    return OracleResult(tokens, logits, p, ids, gap, w, zero_accum, routed, sh, g, total, f64_to_bf16(total))
