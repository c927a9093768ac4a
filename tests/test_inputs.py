"""The seeded input generator: determinism, distributions, and the fp8 weight encoding."""
import numpy as np
import torch

import moe_inputs as mi


def _f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_deterministic_and_offset_consistent():
    a = mi.host_bf16((64, 128), 0, mi.TAG_GATE, 5, mi.SIGMA_W)
    b = mi.host_bf16((64, 128), 0, mi.TAG_GATE, 5, mi.SIGMA_W)
    assert np.array_equal(a, b)
    tail = mi.host_bf16((128,), 0, mi.TAG_GATE, 5, mi.SIGMA_W, first=7 * 128)
    assert np.array_equal(a[7], tail)
    assert not np.array_equal(a, mi.host_bf16((64, 128), 0, mi.TAG_GATE, 6, mi.SIGMA_W))
    assert not np.array_equal(a, mi.host_bf16((64, 128), 1, mi.TAG_GATE, 5, mi.SIGMA_W))
    assert not np.array_equal(a, mi.host_bf16((64, 128), 0, mi.TAG_UP, 5, mi.SIGMA_W))


def test_normal_moments():
    z = mi.host_f32((2_000_000,), 3, mi.TAG_X, 0, 1.0)
    assert abs(z.mean()) < 3e-3 and abs(z.var() - 1.0) < 5e-3
    assert abs(np.mean(z.astype(np.float64) ** 4) - 2.9) < 0.03  # Irwin-Hall(12) kurtosis 3 - 1.2/12
    assert np.abs(z).max() <= 6.0
    w = _f(mi.host_bf16((1_000_000,), 0, mi.TAG_DOWN, 0, mi.SIGMA_W))
    assert abs(w.std() - 0.02) < 2e-4


def test_bf16_fill_is_round_to_nearest_even_of_the_f32_value():
    v = mi.host_f32((100_000,), 0, mi.TAG_UP, 2, mi.SIGMA_W)
    b = mi.host_bf16((100_000,), 0, mi.TAG_UP, 2, mi.SIGMA_W)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_e4m3_weights_reconstruct_within_half_a_code_step():
    q, s = mi.host_e4m3(256, 384, 0, mi.TAG_GATE, 1, mi.SIGMA_W)
    v = mi.host_f32((256 * 384,), 0, mi.TAG_GATE, 1, mi.SIGMA_W).reshape(256, 384).astype(np.float64)
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sc = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)
    err = np.abs(dec * sc - v)
    assert (err <= np.maximum(np.abs(v) * 2.0**-4, sc * 2.0**-10) * 1.0001).all()
    for bi in range(2):
        for bj in range(3):
            blk = v[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            assert s[bi, bj] == np.float32(np.float32(np.abs(blk).max()) / np.float32(448.0))


def test_workload_shapes():
    assert mi.TINY.num_tokens == 16 and mi.TINY.shared_inter == 256
    assert mi.FP8_SIGMOID.weight_dtype == "fp8" and mi.FP8_SIGMOID.routed_scale == 2.5
    assert mi.ZERO_EXPERTS.router_width == 384 and mi.ZERO_EXPERTS.num_experts == 256
    inp = mi.host_inputs(mi.PREFILL_ZIPF.with_tokens(8))
    assert (inp.x[:, 0] == 0x3F80).all()
    perm = mi.expert_permutation(128, 0)
    assert sorted(perm.tolist()) == list(range(128)) and perm[0] != 0
