"""Glue between the seeded workloads of ``moe_inputs`` and the oracle.

TEST INFRASTRUCTURE ONLY.  See ``oracle/__init__.py``.
"""
from __future__ import annotations

import functools
from typing import Optional

import numpy as np

import moe_inputs as mi

from .moe import MoeConfig, OracleResult, moe_forward


def config_of(wl: mi.Workload) -> MoeConfig:
    return MoeConfig(hidden=wl.hidden, num_experts=wl.num_experts, router_width=wl.router_width, top_k=wl.top_k,
                     inter=wl.inter, shared_inter=wl.shared_inter, scoring=wl.scoring,
                     renormalize=wl.renormalize, routed_scale=wl.routed_scale, weight_dtype=wl.weight_dtype)


def run(wl: mi.Workload, tokens: Optional[np.ndarray] = None, layer: int = 0,
        inputs: Optional[mi.HostInputs] = None, expert_cache: Optional[dict] = None,
        forced_ids: Optional[np.ndarray] = None) -> OracleResult:
    """The oracle on workload ``wl`` (all tokens, or the rows ``tokens``), optionally with the
    expert ids of each row given (``forced_ids``, see ``moe_forward``)."""
    inp = inputs if inputs is not None else mi.host_inputs(wl, layer) if tokens is None else None
    if tokens is None:
        x = inp.x
        router, bias = inp.router, inp.bias
    else:
        x = inp.x[tokens] if inp is not None else mi.host_tokens(wl, tokens, layer)
        full = inp if inp is not None else _router_only(wl, layer)
        router, bias = full.router, full.bias
    def expert(e: int):
        if expert_cache is None:
            return mi.host_expert(wl, e, layer)
        if e not in expert_cache:
            expert_cache[e] = mi.host_expert(wl, e, layer)
        return expert_cache[e]

    return moe_forward(config_of(wl), x, router, bias, expert, mi.host_shared(wl, layer), tokens=tokens,
                       shared_gate_bits=mi.host_shared_gate(wl, layer), forced_ids=forced_ids)


@functools.lru_cache(maxsize=8)
def _router_only(wl: mi.Workload, layer: int) -> mi.HostInputs:
    seed = wl.seed + layer
    router = mi.host_bf16((wl.router_width, wl.hidden), seed, mi.TAG_ROUTER, 0, mi.SIGMA_W)
    bias = mi.host_f32((wl.router_width,), seed, mi.TAG_BIAS, 0, mi.SIGMA_BIAS) if wl.has_bias else None
    if wl.zipf_s > 0:
        router[: wl.num_experts, 0] = mi.zipf_router_column(wl.num_experts, wl.zipf_s, wl.zipf_tau, seed)
    return mi.HostInputs(wl, np.empty((0, wl.hidden), np.uint16), router, bias)
