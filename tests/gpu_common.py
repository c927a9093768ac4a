"""Shared helpers of the GPU tests: marshalling workloads through the C ABI and
comparing with the oracle at the stated tolerances."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_bias_amd as moe
import moe_inputs as mi

BF16_TOL = 1e-2  # max|gpu - oracle| <= 1e-2 * max|oracle| for bf16 experts
FP8_TOL = 3e-2  # ... and 3e-2 for fp8 experts
NEAR_TIE = 1e-5  # rows whose K-th and (K+1)-th oracle selection scores differ by less are excluded


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not __import__("os").path.exists(moe.LIB_PATH):
        raise RuntimeError("libmoe.so is not built")


def config_of(wl: mi.Workload):
    return moe.make_config(wl.num_tokens, wl.hidden, wl.num_experts, wl.router_width, wl.top_k, wl.inter,
                           wl.shared_inter, wl.scoring, wl.renormalize, wl.routed_scale, wl.weight_dtype)


def weights_of(dl):
    return moe.weights_from_stacked(dl.router, dl.bias, dl.gate, dl.up, dl.down, dl.gate_s, dl.up_s, dl.down_s,
                                    dl.sh_gate, dl.sh_up, dl.sh_down, dl.sh_gate_s, dl.sh_up_s, dl.sh_down_s,
                                    sh_expert_gate=dl.sh_expert_gate)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit array on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def from_bits(b: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(device)


def run_forward(cfg, w, x):
    ws = torch.empty(moe.moe_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    moe.moe_forward(cfg, w, x, out, ws)
    return out, ws


def assert_close(gpu: np.ndarray, ref: np.ndarray, tol: float, what: str):
    scale = np.abs(ref).max()
    err = np.abs(gpu - ref).max() if gpu.size else 0.0
    assert err <= tol * scale, f"{what}: max|gpu-oracle| = {err:.4g} > {tol} * {scale:.4g}"
    return err / scale if scale > 0 else 0.0


def check_routing(gpu_ids: np.ndarray, res, K: int):
    """ids bit-exact except near-tie rows; returns the mask of rows that agree."""
    near = res.gap < NEAR_TIE
    same = (gpu_ids == res.ids).all(axis=1)
    bad = ~same & ~near
    assert not bad.any(), f"ids differ on {bad.sum()} rows that are not near-ties: {np.nonzero(bad)[0][:8]}"
    return same


def assert_sync_clear(ws, L: dict, what: str):
    """The one-launch decode path's counters (the workspace's first bytes, up to its error word) are
    back at zero, and the error word (set if a tile's bounded wait ever expired) is zero."""
    words = ws[L["sync"]:L["sync_error"] + 4].view(torch.int32)
    assert int(words[-1]) == 0, f"{what}: the decode path's error word is set (a bounded wait expired)"
    assert int(words[:-1].abs().sum()) == 0, f"{what}: decode counters not back at zero"
