"""moe_forward_noalloc, the variant of moe_forward whose workspace is the
library's static per-GPU array: on consecutive calls, the second smaller than
the first, its output equals moe_forward's with a workspace of the caller's,
bit for bit (the same kernels run on the same data)."""
import pytest
import torch

import mixture_experts_layer_bias_amd as moe
import moe_inputs as mi
import moe_inputs.device  # noqa: F401  (mi.device)
from tests.gpu_common import config_of, require_gpu, run_forward, weights_of

pytestmark = pytest.mark.gpu

W = mi.Workload
# largest first: a 300-token layer with a gated shared expert (the multi-kernel path), then decode batches
# (the one-launch experts path, whose counters live in the static array), then an fp8 layer
CALLS = [
    W("na300", 300, 2048, 64, 64, 8, 512, 256, "softmax", True, 1.0, "bf16", False, seed=41, shared_gated=True),
    W("na4", 4, 2048, 128, 128, 8, 768, 0, "softmax", True, 1.0, "bf16", False, seed=42),
    W("na2", 2, 512, 32, 40, 6, 256, 128, "sqrtsoftplus", True, 2.0, "bf16", True, seed=43, shared_gated=True),
    W("na_fp8", 40, 512, 16, 16, 4, 256, 128, "sigmoid", True, 2.5, "fp8", True, seed=44),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_noalloc_equals_forward_on_consecutive_calls():
    for rep in range(2):
        for wl in CALLS:
            print(f"\n[case] moe_forward_noalloc {wl.name} ({wl.num_tokens} tokens), pass {rep}", flush=True)
            cfg = config_of(wl)
            assert moe.moe_workspace_size(cfg) <= moe.MOE_NOALLOC_WORKSPACE_BYTES
            dl = mi.device.device_layer(wl)
            w = weights_of(dl)
            ref, _ = run_forward(cfg, w, dl.x)
            out = torch.full_like(dl.x, 7.0)
            moe.moe_forward_noalloc(cfg, w, dl.x, out)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{wl.name} pass {rep}"


def test_noalloc_refuses_a_layer_beyond_its_static_workspace():
    cfg = config_of(mi.PREFILL_ZIPF)  # about 200 MB of workspace
    dl = mi.device.device_layer(mi.TINY)
    w = weights_of(dl)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_noalloc(cfg, w, dl.x, torch.empty_like(dl.x))
    assert e.value.status == moe.MOE_ERR_WORKSPACE and "static" in e.value.message
