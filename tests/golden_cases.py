"""Builds the tensors of the hand-derived worked examples in ``golden/worked_examples.json``."""
import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _bf16_bits(v: float) -> int:
    u = np.array([v], dtype=np.float32).view(np.uint32)[0]
    assert u & 0xFFFF == 0, f"{v} is not exactly representable in bf16"
    return int(u >> 16)


def load():
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        return json.load(f)["examples"]


def tensors(ex):
    """numpy inputs of one example: bf16 as uint16 bit arrays, bias as float32."""
    c = ex["config"]
    H, E, R, I, Is = c["hidden"], c["num_experts"], c["router_width"], c["inter"], c["shared_inter"]
    x = np.zeros((1, H), np.uint16)
    x[0, 0] = _bf16_bits(1.0)
    router = np.zeros((R, H), np.uint16)
    for r, v in enumerate(ex["router_col0"]):
        router[r, 0] = _bf16_bits(v)
    bias = None if ex["bias"] is None else np.array(ex["bias"], np.float32)
    experts = []
    for e in range(E):
        wg = np.zeros((I, H), np.uint16)
        wu = np.zeros((I, H), np.uint16)
        wd = np.zeros((H, I), np.uint16)
        wg[0, 0] = _bf16_bits(1.0)
        wu[0, 0] = _bf16_bits(2.0)
        wd[0, 0] = _bf16_bits(float(e + 1))
        experts.append((wg, wu, wd))
    shared = None
    if ex["shared"] is not None:
        s = ex["shared"]
        sg = np.zeros((Is, H), np.uint16)
        su = np.zeros((Is, H), np.uint16)
        sd = np.zeros((H, Is), np.uint16)
        sg[0, 0] = _bf16_bits(s["gate_00"])
        su[0, 0] = _bf16_bits(s["up_00"])
        sd[1, 0] = _bf16_bits(s["down_10"])
        shared = (sg, su, sd)
    out = np.zeros(H, np.float64)
    for col, v in ex["out_nonzero"].items():
        out[int(col)] = v
    return dict(x=x, router=router, bias=bias, experts=experts, shared=shared, expected_out=out)
