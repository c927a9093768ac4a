"""Device (torch) copies of a workload's seeded inputs, filled on the GPU by the
same generator definition as the host fills (so both are bit-identical).

Expert weights are stacked per kind ([E, I, H] gate/up, [E, H, I] down) in one
allocation each; the library reaches them through per-expert pointer tables.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import (SIGMA_BIAS, SIGMA_W, SIGMA_X, TAG_BIAS, TAG_DOWN, TAG_GATE, TAG_ROUTER, TAG_SH_DOWN,
               TAG_SH_EXPERT_GATE, TAG_SH_GATE, TAG_SH_UP, TAG_UP, TAG_X, Workload, dev_bf16, dev_e4m3, dev_f32,
               dev_mxfp4, zipf_router_column)


@dataclasses.dataclass
class DeviceLayer:
    wl: Workload
    x: torch.Tensor  # [N, H] bf16
    router: torch.Tensor  # [R, H] bf16
    bias: Optional[torch.Tensor]  # [R] f32
    gate: torch.Tensor  # [E, I, H] bf16 or uint8 (e4m3)
    up: torch.Tensor
    down: torch.Tensor  # [E, H, I]
    gate_s: Optional[torch.Tensor] = None  # [E, I/128, H/128] f32
    up_s: Optional[torch.Tensor] = None
    down_s: Optional[torch.Tensor] = None  # [E, H/128, I/128]
    sh_gate: Optional[torch.Tensor] = None
    sh_up: Optional[torch.Tensor] = None
    sh_down: Optional[torch.Tensor] = None
    sh_gate_s: Optional[torch.Tensor] = None
    sh_up_s: Optional[torch.Tensor] = None
    sh_down_s: Optional[torch.Tensor] = None
    sh_expert_gate: Optional[torch.Tensor] = None  # [H] bf16, the shared expert's sigmoid gate row


def _mat(rows, cols, seed, tag, sub, fp8, device):
    if fp8 == "mxfp4":
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=device)
        dev_mxfp4(q, s, rows, cols, seed, tag, sub, SIGMA_W)
        return q, s
    if not fp8:
        t = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
        dev_bf16(t, seed, tag, sub, SIGMA_W)
        return t, None
    q = torch.empty((rows, cols), dtype=torch.uint8, device=device)
    s = torch.empty(((rows + 127) // 128, (cols + 127) // 128), dtype=torch.float32, device=device)
    dev_e4m3(q, s, rows, cols, seed, tag, sub, SIGMA_W)
    return q, s


def _stack(E, rows, cols, seed, tag, fp8, device):
    if fp8 == "mxfp4":
        w = torch.empty((E, rows, cols // 2), dtype=torch.uint8, device=device)
        s = torch.empty((E, rows, cols // 32), dtype=torch.uint8, device=device)
        for e in range(E):
            dev_mxfp4(w[e], s[e], rows, cols, seed, tag, e, SIGMA_W)
        return w, s
    dt = torch.uint8 if fp8 else torch.bfloat16
    w = torch.empty((E, rows, cols), dtype=dt, device=device)
    s = torch.empty((E, (rows + 127) // 128, (cols + 127) // 128), dtype=torch.float32, device=device) if fp8 else None
    for e in range(E):
        if fp8:
            dev_e4m3(w[e], s[e], rows, cols, seed, tag, e, SIGMA_W)
        else:
            dev_bf16(w[e], seed, tag, e, SIGMA_W)
    return w, s


def device_layer(wl: Workload, layer: int = 0, device: str = "cuda", x_only: bool = False) -> DeviceLayer:
    seed = wl.seed + layer
    N, H, E, R, I, Is = wl.num_tokens, wl.hidden, wl.num_experts, wl.router_width, wl.inter, wl.shared_inter
    fp8 = {"bf16": False, "fp8": True, "mxfp4": "mxfp4"}[wl.weight_dtype]
    x = torch.empty((N, H), dtype=torch.bfloat16, device=device)
    dev_bf16(x, seed, TAG_X, 0, SIGMA_X)
    router = torch.empty((R, H), dtype=torch.bfloat16, device=device)
    dev_bf16(router, seed, TAG_ROUTER, 0, SIGMA_W)
    bias = None
    if wl.has_bias:
        bias = torch.empty((R,), dtype=torch.float32, device=device)
        dev_f32(bias, seed, TAG_BIAS, 0, SIGMA_BIAS)
    if wl.zipf_s > 0:
        if N:
            x[:, 0] = 1.0
        col = zipf_router_column(E, wl.zipf_s, wl.zipf_tau, seed).astype(np.int16)
        router[:E, 0] = torch.from_numpy(col).view(torch.bfloat16).to(device)
    gate, gate_s = _stack(E, I, H, seed, TAG_GATE, fp8, device)
    up, up_s = _stack(E, I, H, seed, TAG_UP, fp8, device)
    down, down_s = _stack(E, H, I, seed, TAG_DOWN, fp8, device)
    lay = DeviceLayer(wl, x, router, bias, gate, up, down, gate_s, up_s, down_s)
    if Is:
        lay.sh_gate, lay.sh_gate_s = _mat(Is, H, seed, TAG_SH_GATE, 0, fp8, device)
        lay.sh_up, lay.sh_up_s = _mat(Is, H, seed, TAG_SH_UP, 0, fp8, device)
        lay.sh_down, lay.sh_down_s = _mat(H, Is, seed, TAG_SH_DOWN, 0, fp8, device)
        if wl.shared_gated:
            lay.sh_expert_gate = torch.empty((H,), dtype=torch.bfloat16, device=device)
            dev_bf16(lay.sh_expert_gate, seed, TAG_SH_EXPERT_GATE, 0, SIGMA_W)
    return lay


def device_x(wl: Workload, layer: int = 0, device: str = "cuda") -> torch.Tensor:
    """Only the token rows of a workload (for extra batches of the same layer)."""
    x = torch.empty((wl.num_tokens, wl.hidden), dtype=torch.bfloat16, device=device)
    dev_bf16(x, wl.seed + layer, TAG_X, 0, SIGMA_X)
    if wl.zipf_s > 0 and wl.num_tokens:
        x[:, 0] = 1.0
    return x
