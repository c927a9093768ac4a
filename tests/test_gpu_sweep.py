"""Seeded random layer shapes through moe_forward, against the oracle.

Each case draws its own configuration: 1 to 256 tokens, H up to 2048, 1 to 256
real experts plus up to E / 2 identity (zero-computation) experts, top-1 to
top-12, I and the shared intermediate up to 768, bf16 / fp8 / MXFP4 experts,
softmax / sigmoid / sqrt(softplus) scoring with or without the correction bias,
renormalisation and scale, an ungated or sigmoid-gated shared expert, and the
row-invariant mode.  Expert ids must match the oracle off near-ties and the
outputs must match at the stated tolerances (forward.rs and forward_prefill.rs
pages: the whole layer forward).
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_bias_amd as moe
import moe_inputs as mi
import moe_inputs.device  # noqa: F401
from oracle import workloads as ow

from tests.gpu_common import BF16_TOL, FP8_TOL, assert_close, check_routing, f64, require_gpu, weights_of

pytestmark = pytest.mark.gpu

CASES = 40


def draw_case(case: int, seed0: int = 7000):
    """Configuration of sweep case `case` (seeded; the same on every host)."""
    rng = np.random.default_rng(seed0 + case)
    c = lambda xs: xs[int(rng.integers(len(xs)))]
    E = int(c([1, 2, 3, 5, 8, 16, 31, 64, 128, 256]))
    R = min(1024, E + int(c([0, 0, 0, 1, 4, max(1, E // 2)])))
    K = int(rng.integers(1, min(R, 12) + 1))
    N = int(c([1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 33, 64, 65, 100, 130, 256]))
    H = 128 * int(c([1, 2, 3, 4, 6, 8, 16]))
    I = 128 * int(c([1, 2, 3, 6]))
    Is = 128 * int(c([0, 0, 1, 2]))
    dt = c(["bf16", "bf16", "fp8", "mxfp4"])
    scoring = c(["softmax", "sigmoid", "sqrtsoftplus"])
    renorm, scale, bias = bool(rng.integers(2)), float(c([1.0, 2.5])), bool(rng.integers(2))
    gated = Is > 0 and bool(rng.integers(2))
    row_invariant = bool(rng.integers(4) == 0)
    while N > 1 and N * K * H * (I + Is) > 1.5e9:  # keeps the float64 oracle to about a second
        N //= 2
    wl = mi.Workload(f"sweep{case}", N, H, E, R, K, I, Is, scoring, renorm, scale, dt, bias, seed=seed0 + case,
                     shared_gated=gated)
    return wl, row_invariant


@pytest.mark.parametrize("case", range(CASES))
def test_random_layer_matches_oracle(case):
    require_gpu()
    wl, rinv = draw_case(case)
    N, K = wl.num_tokens, wl.top_k
    print(f"\n[case] sweep {case}: N{N} H{wl.hidden} E{wl.num_experts} R{wl.router_width} K{K} I{wl.inter} "
          f"Is{wl.shared_inter} {wl.weight_dtype} {wl.scoring} renorm {wl.renormalize} scale {wl.routed_scale} "
          f"bias {wl.has_bias} gated {wl.shared_gated} row_invariant {rinv}", flush=True)
    dl = mi.device.device_layer(wl)
    cfg = moe.make_config(N, wl.hidden, wl.num_experts, wl.router_width, K, wl.inter, wl.shared_inter, wl.scoring,
                          wl.renormalize, wl.routed_scale, wl.weight_dtype, row_invariant=rinv)
    ws = torch.empty(moe.moe_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dl.x)
    moe.moe_forward(cfg, weights_of(dl), dl.x, out, ws)
    torch.cuda.synchronize()
    L = moe.moe_workspace_layout(cfg)
    ids = ws[L["topk_ids"]:L["topk_ids"] + 4 * N * K].view(torch.int32).cpu().numpy().reshape(N, K)
    res = ow.run(wl)
    same = check_routing(ids, res, K)
    got = f64(out)
    assert np.isfinite(got).all(), "non-finite output"
    assert_close(got[same], res.out_f64[same], BF16_TOL if wl.weight_dtype == "bf16" else FP8_TOL, "moe_forward")
