"""Pins of the oracle against things other than itself: hand-derived worked
examples, closed forms, invariants, library routines and brute force."""
import math

import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import codecs, moe as om
from oracle import workloads as ow
from tests import golden_cases


# ============================================================================ codecs

def test_bf16_matches_torch_round_to_nearest_even():
    v = np.random.default_rng(0).standard_normal(200_000).astype(np.float32) * np.float32(37.0)
    ours = codecs.f32_to_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rounds_float64_once():
    # 1 + 2^-8 + 2^-30 sits just above the midpoint of 1 and 1 + 2^-7: one rounding
    # goes up; rounding through fp32 first would drop 2^-30 and tie back to 1.0.
    assert codecs.f64_to_bf16(np.array([1 + 2**-8 + 2**-30]))[0] == 0x3F81
    assert codecs.f64_to_bf16(np.array([1 + 2**-8]))[0] == 0x3F80  # exact tie -> even
    assert codecs.f64_to_bf16(np.array([1 + 3 * 2**-8]))[0] == 0x3F82  # tie -> even (up)
    assert codecs.f64_to_bf16(np.array([-2.0]))[0] == 0xC000


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codecs.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    assert np.array_equal(ref[~np.isnan(ref)], ours[~np.isnan(ours)])


def test_e4m3_published_values():
    # OCP 8-bit floating point, E4M3: max normal 448, min normal 2^-6, min subnormal 2^-9, 1.0 = 0x38
    d = codecs.e4m3_decode(np.array([0x7E, 0x08, 0x01, 0x38, 0xB8, 0x00], np.uint8))
    assert list(d) == [448.0, 2.0**-6, 2.0**-9, 1.0, -1.0, 0.0]
    assert np.isnan(codecs.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_encode_matches_torch_in_range_and_saturates_beyond():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(200_000) * np.exp(rng.uniform(-14, 7, 200_000))).astype(np.float32)
    ours = codecs.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inr = np.abs(v) <= 448
    assert np.array_equal(ours[inr], ref[inr])
    big = v[~inr]
    assert len(big) > 0
    assert np.all(codecs.e4m3_decode(ours[~inr]) == np.sign(big) * 448.0)


def test_e4m3_ties_to_even():
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39); 1.1875 between 0x39 and 0x3A
    c = codecs.e4m3_encode(np.array([1.0625, 1.1875, 2.0**-10, 3 * 2.0**-10]))
    assert list(c) == [0x38, 0x3A, 0x00, 0x02]


def test_e4m3_roundtrip_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(codecs.e4m3_encode(codecs.e4m3_decode(codes)), codes)


# ============================================================================ routing

# OCP Microscaling Formats (MX) v1.0, FP4 E2M1: the eight magnitudes of codes 0..7
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_is_the_published_table():
    got = codecs.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert list(got[:8]) == E2M1_MAGNITUDES
    assert list(-got[8:]) == E2M1_MAGNITUDES and all(np.signbit(got[8:]))


def test_e8m0_decode_is_a_power_of_two():
    got = codecs.e8m0_decode(np.array([0, 1, 120, 127, 128, 254, 255], dtype=np.uint8))
    assert list(got[:6]) == [2.0**-127, 2.0**-126, 2.0**-7, 1.0, 2.0, 2.0**127] and np.isnan(got[6])


def _mx_quantize_reference(v: np.ndarray):
    """An independent MXFP4 quantiser (numpy, per row and 32 columns): shared exponent
    floor(log2(amax)) - 2, element = the nearest E2M1 value of v / 2^X with ties to the even
    code, beyond 6 saturating; a zero block gets scale code 127."""
    rows, cols = v.shape
    mags = np.array(E2M1_MAGNITUDES)
    codes = np.zeros((rows, cols), np.uint8)
    scales = np.zeros((rows, cols // 32), np.uint8)
    for r in range(rows):
        for b in range(cols // 32):
            blk = v[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            x = int(np.floor(np.log2(amax))) - 2 if amax > 0 else 0
            scales[r, b] = x + 127
            for j, val in enumerate(blk / 2.0**x):
                d = np.abs(mags - min(abs(val), 6.0))
                best = [c for c in range(8) if d[c] == d.min()]
                c = min(best, key=lambda c: (c % 2, c))  # ties to the even code
                codes[r, 32 * b + j] = c | (8 if np.signbit(val) else 0)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales


def test_mxfp4_inputs_follow_the_recipe_and_round_trip():
    """The generator's MXFP4 matrices equal an independent numpy quantisation of the same
    fp32 values, and dequantise to within half an E2M1 step of them."""
    rows, cols = 12, 96
    v = mi.host_f32((rows * cols,), 3, mi.TAG_GATE, 5, mi.SIGMA_W).reshape(rows, cols)
    q, s = mi.host_mxfp4(rows, cols, 3, mi.TAG_GATE, 5, mi.SIGMA_W)
    rq, rs = _mx_quantize_reference(v)
    assert np.array_equal(s, rs) and np.array_equal(q, rq)
    w = codecs.mxfp4_dequant(q, s)
    step = np.repeat(codecs.e8m0_decode(s), 32, axis=1)  # the E2M1 step is at most 2 units of 2^X
    assert (np.abs(w - v) <= step + 1e-30).all()


def test_softmax_is_torch_softmax_and_shift_invariant():
    lg = np.random.default_rng(2).standard_normal((7, 384)) * 3
    p = om.scores(lg, "softmax")
    ref = torch.softmax(torch.from_numpy(lg), dim=1).numpy()
    assert np.allclose(p, ref, rtol=1e-13, atol=1e-16)
    assert np.allclose(om.scores(lg + 11.0, "softmax"), p, rtol=1e-12)
    assert np.allclose(p.sum(1), 1.0)


def test_sigmoid_is_expit():
    from scipy.special import expit
    lg = np.random.default_rng(3).standard_normal((5, 64)) * 4
    assert np.allclose(om.scores(lg, "sigmoid"), expit(lg), rtol=1e-14)


def test_sqrtsoftplus_is_sqrt_of_torch_softplus_with_closed_forms():
    """sqrt(softplus(z)) against torch's softplus in float64, over a range that
    overflows a naive exp; closed forms at 0 and in both tails."""
    z = np.concatenate([np.linspace(-60.0, 60.0, 241), np.random.default_rng(31).standard_normal(200) * 4])
    ref = torch.sqrt(torch.nn.functional.softplus(torch.from_numpy(z), threshold=1000.0)).numpy()
    got = om.scores(z[None, :], "sqrtsoftplus")[0]
    assert np.allclose(got, ref, rtol=1e-14, atol=0)
    edge = om.scores(np.array([[0.0, 800.0, -800.0, 30.0, -30.0]]), "sqrtsoftplus")[0]
    assert edge[0] == pytest.approx(math.sqrt(math.log(2.0)), rel=1e-15)
    assert edge[1] == pytest.approx(math.sqrt(800.0), rel=1e-15)  # softplus(z) -> z
    assert edge[2] == 0.0 or edge[2] < 1e-170  # softplus(z) -> e^z, so the score -> e^(z/2)
    assert edge[3] == pytest.approx(math.sqrt(30.0 + math.exp(-30.0)), rel=1e-15)
    assert edge[4] == pytest.approx(math.exp(-15.0), rel=1e-12)


def test_sqrtsoftplus_without_bias_selects_topk_of_logits_and_renormalises():
    """sqrt(softplus) is increasing, so without a bias the K best scores are the K
    best logits; renormalised weights sum to 1, then times the scale."""
    lg = np.random.default_rng(32).standard_normal((40, 64)) * 3
    p = om.scores(lg, "sqrtsoftplus")
    ids, _ = om.select_topk(p, None, 6)
    assert np.array_equal(ids, np.argsort(-lg, axis=1, kind="stable")[:, :6])
    w, _ = om.routing_weights(p, ids, True, 2.0, 64)
    assert np.allclose(w.sum(1), 2.0, rtol=1e-14)


def test_topk_equals_full_sort_brute_force_with_ties():
    rng = np.random.default_rng(4)
    p = rng.integers(0, 6, size=(200, 12)).astype(np.float64) / 8.0  # many exact ties
    bias = rng.integers(-2, 3, size=12).astype(np.float32) / 8.0
    ids, gap = om.select_topk(p, bias, 4)
    for t in range(p.shape[0]):
        s = [p[t, r] + float(bias[r]) for r in range(12)]
        order = sorted(range(12), key=lambda r: (-s[r], r))  # larger first, then lower index
        assert list(ids[t]) == order[:4]
        assert gap[t] == s[order[3]] - s[order[4]]


def test_sigmoid_without_bias_selects_topk_of_logits():
    lg = np.random.default_rng(5).standard_normal((50, 32))
    ids, _ = om.select_topk(om.scores(lg, "sigmoid"), None, 5)
    ref = np.argsort(-lg, axis=1, kind="stable")[:, :5]
    assert np.array_equal(ids, ref)


def test_dominant_column_gives_one_hot():
    lg = np.zeros((3, 16))
    lg[:, 9] = 50.0
    p = om.scores(lg, "softmax")
    ids, _ = om.select_topk(p, None, 1)
    w, z = om.routing_weights(p, ids, True, 1.0, 16)
    assert (ids[:, 0] == 9).all() and np.allclose(w, 1.0) and (z == 0).all()


def test_weights_sum_to_one_after_renorm_and_to_scale():
    lg = np.random.default_rng(6).standard_normal((64, 128))
    p = om.scores(lg, "softmax")
    ids, _ = om.select_topk(p, None, 8)
    w, _ = om.routing_weights(p, ids, True, 1.0, 128)
    assert np.allclose(w.sum(1), 1.0, rtol=1e-14)
    ps = om.scores(lg, "sigmoid")
    ids, _ = om.select_topk(ps, np.full(128, 0.1, np.float32), 8)
    w, _ = om.routing_weights(ps, ids, True, 2.5, 128)
    assert np.allclose(w.sum(1), 2.5, rtol=1e-14)
    # weights are the UNBIASED scores of the selected columns, in slot order
    ratio = w / np.take_along_axis(ps, ids.astype(np.int64), 1)
    assert np.allclose(ratio, ratio[:, :1])


def test_k_equals_r_gives_the_full_softmax_mixture():
    lg = np.random.default_rng(7).standard_normal((9, 8))
    p = om.scores(lg, "softmax")
    ids, gap = om.select_topk(p, None, 8)
    w, _ = om.routing_weights(p, ids, True, 1.0, 8)
    dense = np.zeros_like(p)
    np.put_along_axis(dense, ids.astype(np.int64), w, 1)
    assert np.allclose(dense, p, rtol=1e-14) and np.isinf(gap).all()


def test_zero_accum_is_the_identity_expert_weight_and_unrenormalised_sum_below_one():
    lg = np.random.default_rng(8).standard_normal((40, 24))
    p = om.scores(lg, "softmax")
    bias = np.random.default_rng(9).standard_normal(24).astype(np.float32) * 0.1
    ids, _ = om.select_topk(p, bias, 6)
    w, z = om.routing_weights(p, ids, False, 1.0, 16)
    for t in range(40):
        assert z[t] == pytest.approx(sum(p[t, r] for r in ids[t] if r >= 16), rel=1e-14, abs=0)
    assert (w.sum(1) < 1.0).all()


# ============================================================================ sort by expert

def test_sort_by_expert_is_a_stable_bijection():
    ids = np.random.default_rng(10).integers(0, 40, size=(300, 6)).astype(np.int32)
    counts, offsets, sorted_ids, inv = om.sort_by_expert(ids, 40)
    flat = ids.reshape(-1)
    assert counts.sum() == flat.size and offsets[-1] == flat.size and offsets[0] == 0
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(inv[sorted_ids], np.arange(flat.size))  # bijection
    assert np.array_equal(sorted_ids, np.argsort(flat, kind="stable"))  # library stable sort
    for e in range(40):
        assert (flat[sorted_ids[offsets[e]:offsets[e + 1]]] == e).all()
    assert np.array_equal(counts, np.bincount(flat, minlength=40))


# ============================================================================ fp8 activations

def test_quantize_fp8_groups_hand_example():
    v = np.zeros((2, 256), np.float32)
    v[0, :4] = [1.0, -0.5, 0.25, 3.5]  # amax 3.5 -> inv 128, scale 3.5/448 = 1/128
    v[0, 128] = 7.0  # second group: amax 7 -> inv 64
    q, s = om.quantize_fp8_groups(v)
    assert s[0, 0] == np.float32(3.5 / 448) and s[0, 1] == np.float32(7.0 / 448)
    assert s[1, 0] == 1.0 and s[1, 1] == 1.0 and (q[1] == 0).all()  # zero groups
    d = om.dequant_rows(q, s)
    assert list(d[0, :4]) == [1.0, -0.5, 0.25, 3.5] and d[0, 128] == 7.0
    assert q[0, 3] == 0x7E  # amax maps onto 448


def test_quantize_fp8_groups_matches_per_element_torch_and_error_bound():
    x = (np.random.default_rng(11).standard_normal((16, 512)) * 3).astype(np.float32)
    q, s = om.quantize_fp8_groups(x)
    g = x.reshape(16, 4, 128)
    amax = np.abs(g).max(2)
    inv = (np.float32(448.0) / amax).astype(np.float32)
    ref = torch.from_numpy((g * inv[:, :, None]).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(q, ref.numpy().reshape(16, 512))
    err = np.abs(om.dequant_rows(q, s) - x)
    bound = np.maximum(np.abs(x) * 2.0**-4, np.repeat(s, 128, 1) * 2.0**-10) * (1 + 1e-6)
    assert (err <= bound).all()


# ============================================================================ experts

def _bf16(a):
    return codecs.f64_to_bf16(np.asarray(a, np.float64))


def test_single_expert_top1_is_a_plain_swiglu_mlp():
    """E = 1, K = 1, renormalised: the layer is SwiGLU-MLP(x) (torch float64 + F.silu)."""
    rng = np.random.default_rng(12)
    N, H, I = 5, 64, 32
    x, wr = _bf16(rng.standard_normal((N, H))), _bf16(rng.standard_normal((1, H)) * 0.1)
    wg, wu, wd = (_bf16(rng.standard_normal(s) * 0.1) for s in ((I, H), (I, H), (H, I)))
    cfg = om.MoeConfig(H, 1, 1, 1, I, 0, "softmax", True, 1.0, "bf16")
    res = om.moe_forward(cfg, x, wr, None, lambda e: (wg, wu, wd), None)
    t = lambda b: torch.from_numpy(codecs.bf16_to_f64(b))
    h = torch.nn.functional.silu(t(x) @ t(wg).T) * (t(x) @ t(wu).T)
    # torch rounds float64 -> bf16 through fp32 (a rare double rounding), so h may
    # differ by one bf16 ulp in a few places: compare with a tolerance, not bits.
    h = h.to(torch.bfloat16).to(torch.float64)
    y = h @ t(wd).T
    assert np.abs(res.out_f64 - y.numpy()).max() <= 1e-3 * float(y.abs().max())
    assert (res.ids == 0).all() and np.allclose(res.weights, 1.0)


def _dense_brute_force(cfg, x_bits, router_bits, bias, experts, shared, shared_gate_bits=None):
    """North-star brute force: a per-token loop over ALL experts, gates zeroed
    unless selected; written with Python loops and a full sort per token."""
    out = []
    E, R, K = cfg.num_experts, cfg.router_width, cfg.top_k
    X = codecs.bf16_to_f64(x_bits)
    Wr = codecs.bf16_to_f64(router_bits)
    for t in range(X.shape[0]):
        logit = [float(np.dot(X[t], Wr[r])) for r in range(R)]
        if cfg.scoring == "softmax":
            m = max(logit)
            ex = [math.exp(v - m) for v in logit]
            p = [v / sum(ex) for v in ex]
        elif cfg.scoring == "sigmoid":
            p = [1 / (1 + math.exp(-v)) for v in logit]
        else:  # sqrt(softplus), softplus(v) = ln(1 + e^v)
            p = [math.sqrt(math.log1p(math.exp(v))) for v in logit]
        sel = [p[r] + (float(bias[r]) if bias is not None else 0.0) for r in range(R)]
        chosen = sorted(range(R), key=lambda r: (-sel[r], r))[:K]
        denom = sum(p[r] for r in chosen) if cfg.renormalize else 1.0
        gate = [0.0] * R
        for r in chosen:
            gate[r] = p[r] / denom * cfg.routed_scale
        acc = np.zeros(cfg.hidden)
        for e in range(E):  # every expert, selected or not
            if cfg.weight_dtype == "bf16":
                wg, wu, wd = (codecs.bf16_to_f64(w) for w in experts[e])
                g, u = wg @ X[t], wu @ X[t]
                h = codecs.bf16_to_f64(codecs.f64_to_bf16(g / (1 + np.exp(-g)) * u))
                y = wd @ h
            else:
                y = _fp8_expert_blockwise(X[t], experts[e])
            acc += gate[e] * y
        for r in range(E, R):
            acc += gate[r] * X[t]
        if shared is not None:
            gsh = 1.0
            if shared_gate_bits is not None:
                gv = codecs.bf16_to_f64(shared_gate_bits)
                gsh = 1 / (1 + math.exp(-sum(float(X[t, i]) * float(gv[i]) for i in range(cfg.hidden))))
            if cfg.weight_dtype == "bf16":
                sg, su, sd = (codecs.bf16_to_f64(w) for w in shared)
                g, u = sg @ X[t], su @ X[t]
                acc += gsh * (sd @ codecs.bf16_to_f64(codecs.f64_to_bf16(g / (1 + np.exp(-g)) * u)))
            else:
                acc += gsh * _fp8_expert_blockwise(X[t], shared)
        out.append(acc)
    return np.array(out)


def _fp8_expert_blockwise(xrow, w):
    """One row through an fp8 or MXFP4 expert, as sums over 128-blocks of the activation:
    s_x * S_w * (code dot product) for e4m3 weights with 128x128 block scales, or
    s_x * sum over the four 32-column weight blocks of 2^(e - 127) * (code dot product) for
    MXFP4 weights (E2M1 codes unpacked from their nibbles)."""
    (qg, sg), (qu, su), (qd, sd) = w
    xq, xs = om.quantize_fp8_groups(xrow[None, :].astype(np.float32))

    def gemv(codes, scales, aq, as_):
        mx = scales.dtype == np.uint8
        out = np.zeros(codes.shape[0])
        for i in range(codes.shape[0]):
            if mx:
                wrow = np.empty(codes.shape[1] * 2, np.uint8)
                wrow[0::2], wrow[1::2] = codes[i] & 0xF, codes[i] >> 4
            tot = 0.0
            for b in range(aq.shape[1] // 128):
                a = codecs.e4m3_decode(aq[0, b * 128:(b + 1) * 128])
                if mx:
                    inner = 0.0
                    for j in range(4):
                        k0 = b * 128 + 32 * j
                        inner += 2.0 ** (int(scales[i, k0 // 32]) - 127) * float(
                            np.dot(codecs.e2m1_decode(wrow[k0:k0 + 32]), a[32 * j:32 * j + 32]))
                    tot += float(as_[0, b]) * inner
                else:
                    dot = float(np.dot(codecs.e4m3_decode(codes[i, b * 128:(b + 1) * 128]), a))
                    tot += float(as_[0, b]) * float(scales[i // 128, b]) * dot
            out[i] = tot
        return out

    g, u = gemv(qg, sg, xq, xs), gemv(qu, su, xq, xs)
    hq, hs = om.quantize_fp8_groups((g / (1 + np.exp(-g)) * u)[None, :].astype(np.float32))
    return gemv(qd, sd, hq, hs)


def _random_layer(rng, N, H, E, R, K, I, Is, scoring, renorm, scale, dtype, with_bias):
    x = _bf16(rng.standard_normal((N, H)))
    wr = _bf16(rng.standard_normal((R, H)) * 0.2)
    bias = (rng.standard_normal(R) * 0.1).astype(np.float32) if with_bias else None

    def mk(rows, cols):
        w = rng.standard_normal((rows, cols)) * 0.05
        if dtype == "bf16":
            return _bf16(w)
        if dtype == "mxfp4":
            return _mx_quantize_reference(w.astype(np.float32))
        s = np.zeros(((rows + 127) // 128, (cols + 127) // 128), np.float32)
        q = np.zeros((rows, cols), np.uint8)
        for bi in range(s.shape[0]):
            for bj in range(s.shape[1]):
                blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
                s[bi, bj] = np.float32(np.abs(blk).max() / 448.0)
                q[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128] = codecs.e4m3_encode(
                    blk.astype(np.float32) / s[bi, bj])
        return q, s

    experts = [(mk(I, H), mk(I, H), mk(H, I)) for _ in range(E)]
    shared = (mk(Is, H), mk(Is, H), mk(H, Is)) if Is else None
    cfg = om.MoeConfig(H, E, R, K, I, Is, scoring, renorm, scale, dtype)
    return cfg, x, wr, bias, experts, shared


@pytest.mark.parametrize("case", [
    dict(N=6, H=32, E=8, R=8, K=2, I=16, Is=24, scoring="softmax", renorm=True, scale=1.0, dtype="bf16",
         with_bias=False),
    dict(N=5, H=32, E=6, R=6, K=3, I=16, Is=0, scoring="sigmoid", renorm=True, scale=2.5, dtype="bf16",
         with_bias=True),
    dict(N=7, H=32, E=6, R=10, K=4, I=16, Is=0, scoring="softmax", renorm=False, scale=1.0, dtype="bf16",
         with_bias=True),
    dict(N=3, H=256, E=4, R=4, K=2, I=128, Is=128, scoring="sigmoid", renorm=True, scale=2.5, dtype="fp8",
         with_bias=True),
    dict(N=6, H=32, E=8, R=8, K=3, I=16, Is=0, scoring="sqrtsoftplus", renorm=True, scale=1.5, dtype="bf16",
         with_bias=True),
    dict(N=5, H=32, E=6, R=9, K=3, I=16, Is=24, scoring="sqrtsoftplus", renorm=False, scale=1.0, dtype="bf16",
         with_bias=True, gated=True),
    dict(N=3, H=256, E=4, R=4, K=2, I=128, Is=128, scoring="softmax", renorm=True, scale=1.0, dtype="fp8",
         with_bias=False, gated=True),
    dict(N=3, H=256, E=4, R=6, K=3, I=128, Is=128, scoring="sqrtsoftplus", renorm=True, scale=2.5, dtype="mxfp4",
         with_bias=True, gated=True),
])
def test_oracle_equals_dense_brute_force(case):
    rng = np.random.default_rng(13)
    case = dict(case)
    gated = case.pop("gated", False)
    cfg, x, wr, bias, experts, shared = _random_layer(rng, **case)
    gate = _bf16(rng.standard_normal(cfg.hidden) * 0.2) if gated else None
    res = om.moe_forward(cfg, x, wr, bias, lambda e: experts[e], shared, shared_gate_bits=gate)
    ref = _dense_brute_force(cfg, x, wr, bias, experts, shared, gate)
    assert np.allclose(res.out_f64, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())
    assert np.array_equal(res.out_bits, codecs.f64_to_bf16(ref)) or np.abs(
        codecs.bf16_to_f64(res.out_bits) - codecs.bf16_to_f64(codecs.f64_to_bf16(ref))).max() <= \
        2**-8 * np.abs(ref).max()


def test_identity_experts_only_closed_form():
    """A bias that forces every slot onto identity experts (columns E..R-1, the
    first one included): out = bf16((sum of the chosen softmax scores) * x)."""
    rng = np.random.default_rng(14)
    cfg, x, wr, _, experts, _ = _random_layer(rng, 9, 32, 4, 8, 4, 16, 0, "softmax", False, 1.0, "bf16", False)
    bias = np.zeros(8, np.float32)
    bias[4:] = 10.0  # K = 4 = R - E: all four identity columns are chosen
    res = om.moe_forward(cfg, x, wr, bias, lambda e: experts[e], None)
    X = torch.from_numpy(codecs.bf16_to_f64(x))
    p = torch.softmax(X @ torch.from_numpy(codecs.bf16_to_f64(wr)).T, dim=1)
    expected = (p[:, 4:].sum(1, keepdim=True) * X).numpy()
    assert (np.sort(res.ids, 1) == np.arange(4, 8)).all()
    assert np.abs(codecs.bf16_to_f64(res.out_bits) - expected).max() <= 2**-8 * np.abs(expected).max()
    assert np.allclose(res.zero_accum, p[:, 4:].sum(1).numpy(), rtol=1e-14)


def test_first_identity_column_counts_as_identity():
    """Column E exactly is the first zero-computation expert."""
    p = np.full((1, 6), 1 / 6)
    ids = np.array([[4, 0]], np.int32)
    w, z = om.routing_weights(p, ids, False, 1.0, 4)
    assert z[0] == pytest.approx(1 / 6, rel=1e-15)


def test_zero_routed_down_leaves_the_shared_expert():
    rng = np.random.default_rng(15)
    cfg, x, wr, bias, experts, shared = _random_layer(rng, 4, 32, 4, 4, 2, 16, 32, "softmax", True, 1.0, "bf16",
                                                      False)
    zero = [(g, u, np.zeros_like(d)) for g, u, d in experts]
    res = om.moe_forward(cfg, x, wr, bias, lambda e: zero[e], shared)
    sg, su, sd = (codecs.bf16_to_f64(w) for w in shared)
    X = codecs.bf16_to_f64(x)
    g, u = X @ sg.T, X @ su.T
    ref = codecs.bf16_to_f64(codecs.f64_to_bf16(torch.nn.functional.silu(torch.from_numpy(g)).numpy() * u)) @ sd.T
    assert np.allclose(res.out_f64, ref, rtol=1e-12)


def test_shared_gate_closed_forms():
    """A zero gate row weighs the shared expert by sigmoid(0) = 1/2 exactly, which
    equals the ungated layer with the shared W_down halved (exact in bf16).  For
    one token, a gate row of 8 x (resp. -8 x) saturates the sigmoid to exactly 1
    (resp. 0) in float64: the ungated layer, resp. the layer with no shared expert."""
    rng = np.random.default_rng(33)
    cfg, x, wr, bias, experts, shared = _random_layer(rng, 1, 64, 4, 4, 2, 16, 32, "softmax", True, 1.0, "bf16",
                                                      False)
    ex = lambda e: experts[e]
    ungated = om.moe_forward(cfg, x, wr, bias, ex, shared)
    half = (shared[0], shared[1], _bf16(codecs.bf16_to_f64(shared[2]) * 0.5))
    a = om.moe_forward(cfg, x, wr, bias, ex, shared, shared_gate_bits=np.zeros(64, np.uint16))
    b = om.moe_forward(cfg, x, wr, bias, ex, half)
    assert np.array_equal(a.out_f64, b.out_f64) and (a.shared_weight == 0.5).all()
    up = om.moe_forward(cfg, x, wr, bias, ex, shared, shared_gate_bits=_bf16(codecs.bf16_to_f64(x[0]) * 8))
    assert np.array_equal(up.out_f64, ungated.out_f64)
    cfg0 = om.MoeConfig(cfg.hidden, cfg.num_experts, cfg.router_width, cfg.top_k, cfg.inter, 0, cfg.scoring,
                        cfg.renormalize, cfg.routed_scale, cfg.weight_dtype)
    down = om.moe_forward(cfg, x, wr, bias, ex, shared, shared_gate_bits=_bf16(codecs.bf16_to_f64(x[0]) * -8))
    assert np.array_equal(down.out_f64, om.moe_forward(cfg0, x, wr, bias, ex, None).out_f64)


def test_routed_part_is_linear_in_w_down():
    rng = np.random.default_rng(16)
    cfg, x, wr, bias, experts, _ = _random_layer(rng, 6, 32, 6, 6, 2, 16, 0, "softmax", True, 1.0, "bf16", False)
    doubled = [(g, u, _bf16(codecs.bf16_to_f64(d) * 2)) for g, u, d in experts]  # exact in bf16
    a = om.moe_forward(cfg, x, wr, bias, lambda e: experts[e], None)
    b = om.moe_forward(cfg, x, wr, bias, lambda e: doubled[e], None)
    assert np.allclose(b.routed, 2 * a.routed, rtol=1e-14, atol=0)


def test_fp8_expert_dequantised_gemm_equals_blockwise_sum():
    rng = np.random.default_rng(17)
    cfg, x, _, _, experts, _ = _random_layer(rng, 2, 256, 1, 1, 1, 256, 0, "softmax", True, 1.0, "fp8", False)
    X = codecs.bf16_to_f64(x)
    xq, xs = om.quantize_fp8_groups(X.astype(np.float32))
    y = om.swiglu_expert_fp8(xq, xs, *experts[0])
    for t in range(2):
        assert np.allclose(y[t], _fp8_expert_blockwise(X[t], experts[0]), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("ex", golden_cases.load(), ids=lambda e: e["name"])
def test_hand_derived_worked_examples(ex):
    g = golden_cases.tensors(ex)
    c = ex["config"]
    cfg = om.MoeConfig(c["hidden"], c["num_experts"], c["router_width"], c["top_k"], c["inter"],
                       c["shared_inter"], c["scoring"], c["renormalize"], c["routed_scale"], "bf16")
    res = om.moe_forward(cfg, g["x"], g["router"], g["bias"], lambda e: g["experts"][e], g["shared"])
    assert list(res.ids[0]) == ex["ids"]
    assert np.allclose(res.weights[0], ex["weights"], rtol=1e-13)
    assert res.zero_accum[0] == pytest.approx(ex["zero_accum"], rel=1e-13, abs=1e-300)
    assert np.array_equal(codecs.bf16_to_f64(res.out_bits[0]), g["expected_out"])


# ============================================================================ workloads

def test_prefill_workload_loads_are_zipf_skewed():
    """The skewed-router recipe gives a log-log slope near -1.1 over the expert loads."""
    wl = mi.PREFILL_ZIPF
    inp = mi.host_inputs(wl)
    p = om.scores(om.router_logits(inp.x, inp.router), "softmax")
    ids, gap = om.select_topk(p, None, wl.top_k)
    loads = np.sort(np.bincount(ids.ravel(), minlength=wl.num_experts))[::-1]
    assert loads.sum() == wl.num_tokens * wl.top_k and (loads > 0).all()
    ranks = np.arange(1, len(loads) + 1)
    sel = slice(0, 64)  # unsaturated ranks
    slope = np.polyfit(np.log(ranks[sel]), np.log(loads[sel]), 1)[0]
    assert -1.4 < slope < -0.8, slope
    assert (gap < 1e-5).sum() < 0.02 * wl.num_tokens


def test_tiny_workload_smoke_and_invariants():
    res = ow.run(mi.TINY)
    assert res.out_bits.shape == (16, 256)
    assert np.allclose(res.weights.sum(1), 1.0)
    c, o, s, i = om.sort_by_expert(res.ids, mi.TINY.router_width)
    assert c.sum() == 32 and np.array_equal(i[s], np.arange(32))
