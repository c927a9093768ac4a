"""Seeded synthetic inputs for the MoE layer forward.

Holds the five workload shapes, the counter-based generator (``gen_core.h``,
compiled for the host by gcc and for gfx950 by hipcc so both fills are
bit-identical) and the skewed-router construction of the prefill workload.
Nothing here computes any step of the MoE forward: the oracle and the HIP
library each implement the method on their own and only share these inputs.

bf16 tensors are handled on the host as ``numpy.uint16`` bit patterns and e4m3
tensors as ``numpy.uint8`` codes.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libmoe_inputs_host.so")
DEV_LIB = os.path.join(_HERE, "libmoe_inputs_dev.so")

TAG_X, TAG_ROUTER, TAG_BIAS, TAG_GATE, TAG_UP, TAG_DOWN = 1, 2, 3, 4, 5, 6
TAG_SH_GATE, TAG_SH_UP, TAG_SH_DOWN, TAG_PERM, TAG_SH_EXPERT_GATE = 7, 8, 9, 10, 11

SIGMA_X = 1.0
SIGMA_W = 0.02
SIGMA_BIAS = 0.1


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and routing recipe of one MoE layer workload."""

    name: str
    num_tokens: int  # N
    hidden: int  # H
    num_experts: int  # E real SwiGLU experts
    router_width: int  # R >= E; columns [E, R) are identity (zero-computation) experts
    top_k: int  # K
    inter: int  # I
    shared_inter: int  # Is, 0 = no shared expert
    scoring: str  # "softmax" | "sigmoid" | "sqrtsoftplus"
    renormalize: bool
    routed_scale: float
    weight_dtype: str  # "bf16" | "fp8" | "mxfp4"
    has_bias: bool
    zipf_s: float = 0.0  # > 0: skewed router column (prefill workload)
    zipf_tau: float = 0.0
    seed: int = 0
    shared_gated: bool = False  # the shared expert has a sigmoid gate (one weight row [H])

    def with_tokens(self, n: int) -> "Workload":
        return dataclasses.replace(self, num_tokens=n)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  Names say what each is.
TINY = Workload("tiny_16tok_h256_e8_top2_shared256", 16, 256, 8, 8, 2, 128, 256, "softmax", True, 1.0,
                "bf16", False)
DECODE = Workload("decode_4tok_h2048_e128_top8_i768", 4, 2048, 128, 128, 8, 768, 0, "softmax", True, 1.0,
                  "bf16", False)
PREFILL_ZIPF = Workload("prefill_4096tok_h2048_e128_top8_i768_zipf1.1", 4096, 2048, 128, 128, 8, 768, 0,
                        "softmax", True, 1.0, "bf16", False, zipf_s=1.1, zipf_tau=0.5)
FP8_SIGMOID = Workload("fp8_2048tok_h7168_e256_top8_i2048_shared2048_sigmoid_bias", 2048, 7168, 256, 256, 8, 2048,
                       2048, "sigmoid", True, 2.5, "fp8", True)
ZERO_EXPERTS = Workload("zero_experts_512tok_h6144_e256+128id_top12_i2048", 512, 6144, 256, 384, 12, 2048, 0,
                        "softmax", False, 1.0, "bf16", True)
# The DeepSeek-like layer with MXFP4 experts (E2M1 codes, E8M0 scales per 32 columns), fp8 activations.
MXFP4_SIGMOID = Workload("mxfp4_2048tok_h7168_e256_top8_i2048_shared2048_sigmoid_bias", 2048, 7168, 256, 256, 8,
                         2048, 2048, "sigmoid", True, 2.5, "mxfp4", True)

WORKLOADS = {"tiny": TINY, "decode": DECODE, "prefill_zipf": PREFILL_ZIPF, "fp8_sigmoid": FP8_SIGMOID,
             "zero_experts": ZERO_EXPERTS, "mxfp4_sigmoid": MXFP4_SIGMOID}


# ----------------------------------------------------------------------------- build

def _gcc_cmd(out: str) -> list:
    return ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-ffp-contract=off",
            os.path.join(_HERE, "gen_host.c"), "-o", out]


def _hipcc_cmd(out: str) -> list:
    return ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            os.path.join(_HERE, "gen_device.hip"), "-o", out]


def build(device: bool = True) -> None:
    """Compile the host generator (gcc) and, if ``device``, the gfx950 one (hipcc)."""
    for cmd, out in ((_gcc_cmd, HOST_LIB), (_hipcc_cmd, DEV_LIB)):
        if out == DEV_LIB and not device:
            continue
        tmp = out + ".tmp"
        subprocess.run(cmd(tmp), check=True, cwd=_HERE)
        os.replace(tmp, out)


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build(device=False)
        lib = ctypes.CDLL(HOST_LIB)
        u64, u32, f32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p
        lib.mi_host_fill_bf16.argtypes = [vp, u64, u64, u64, u32, u32, f32]
        lib.mi_host_fill_f32.argtypes = [vp, u64, u64, u64, u32, u32, f32]
        lib.mi_host_fill_e4m3.argtypes = [vp, vp, u32, u32, u64, u32, u32, f32]
        lib.mi_host_fill_mxfp4.argtypes = [vp, vp, u32, u32, u64, u32, u32, f32]
        for f in (lib.mi_host_fill_bf16, lib.mi_host_fill_f32, lib.mi_host_fill_e4m3, lib.mi_host_fill_mxfp4):
            f.restype = None
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run moe_inputs.build()")
        lib = ctypes.CDLL(DEV_LIB)
        u64, u32, f32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p
        lib.mi_dev_fill_bf16.argtypes = [vp, u64, u64, u64, u32, u32, f32, vp]
        lib.mi_dev_fill_f32.argtypes = [vp, u64, u64, u64, u32, u32, f32, vp]
        lib.mi_dev_fill_e4m3.argtypes = [vp, vp, u32, u32, u64, u32, u32, f32, vp]
        lib.mi_dev_fill_mxfp4.argtypes = [vp, vp, u32, u32, u64, u32, u32, f32, vp]
        for f in (lib.mi_dev_fill_bf16, lib.mi_dev_fill_f32, lib.mi_dev_fill_e4m3, lib.mi_dev_fill_mxfp4):
            f.restype = ctypes.c_int
        _dev = lib
    return _dev


# ----------------------------------------------------------------------------- host fills

def host_bf16(shape, seed: int, tag: int, sub: int, sigma: float, first: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    _host_lib().mi_host_fill_bf16(out.ctypes.data, n, first, seed, tag, sub, sigma)
    return out.reshape(shape)


def host_f32(shape, seed: int, tag: int, sub: int, sigma: float, first: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    _host_lib().mi_host_fill_f32(out.ctypes.data, n, first, seed, tag, sub, sigma)
    return out.reshape(shape)


def host_e4m3(rows: int, cols: int, seed: int, tag: int, sub: int, sigma: float):
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty(((rows + 127) // 128, (cols + 127) // 128), dtype=np.float32)
    _host_lib().mi_host_fill_e4m3(q.ctypes.data, s.ctypes.data, rows, cols, seed, tag, sub, sigma)
    return q, s


def host_mxfp4(rows: int, cols: int, seed: int, tag: int, sub: int, sigma: float):
    """MXFP4 matrix: (packed E2M1 codes uint8 [rows, cols/2], E8M0 scale codes uint8 [rows, cols/32])."""
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    s = np.empty((rows, cols // 32), dtype=np.uint8)
    _host_lib().mi_host_fill_mxfp4(q.ctypes.data, s.ctypes.data, rows, cols, seed, tag, sub, sigma)
    return q, s


# ----------------------------------------------------------------------------- skewed router

def _bf16_bits_host(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits via float32 (round to nearest even at each step)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def expert_permutation(num_experts: int, seed: int) -> np.ndarray:
    """A seeded permutation of expert ids (sort by a hash of (seed, expert))."""
    keys = np.array([_py_mix64(_py_mix64(seed + 0x9E3779B97F4A7C15 * (TAG_PERM + 1)) ^ e) for e in
                     range(num_experts)], dtype=np.uint64)
    return np.argsort(keys, kind="stable").astype(np.int64)


def _py_mix64(z: int) -> int:
    m = (1 << 64) - 1
    z &= m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


def zipf_router_column(num_experts: int, s: float, tau: float, seed: int) -> np.ndarray:
    """bf16 bits of column 0 of the router for the skewed-load workload.

    Every token's channel 0 is 1.0, so this column adds tau*ln(p_rank) to the
    logit of the expert holding that load rank, with p_rank proportional to
    rank^-s.  A seeded permutation decides which expert gets which rank, so the
    hot experts are not the low ids.
    """
    ranks = np.arange(1, num_experts + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    perm = expert_permutation(num_experts, seed)
    col = np.empty(num_experts, dtype=np.float64)
    col[perm] = tau * np.log(p)
    return _bf16_bits_host(col)


# ----------------------------------------------------------------------------- whole workloads (host)

@dataclasses.dataclass
class HostInputs:
    """Host copies of the inputs that every workload has (experts are fetched lazily)."""

    wl: Workload
    x: np.ndarray  # [N, H] bf16 bits
    router: np.ndarray  # [R, H] bf16 bits
    bias: Optional[np.ndarray]  # [R] f32 or None


def host_inputs(wl: Workload, layer: int = 0) -> HostInputs:
    seed = wl.seed + layer
    x = host_bf16((wl.num_tokens, wl.hidden), seed, TAG_X, 0, SIGMA_X)
    router = host_bf16((wl.router_width, wl.hidden), seed, TAG_ROUTER, 0, SIGMA_W)
    bias = host_f32((wl.router_width,), seed, TAG_BIAS, 0, SIGMA_BIAS) if wl.has_bias else None
    if wl.zipf_s > 0:
        x[:, 0] = 0x3F80  # exactly 1.0
        router[: wl.num_experts, 0] = zipf_router_column(wl.num_experts, wl.zipf_s, wl.zipf_tau, seed)
    return HostInputs(wl, x, router, bias)


def host_tokens(wl: Workload, tokens: np.ndarray, layer: int = 0) -> np.ndarray:
    """Rows ``tokens`` of x, generated directly (no need to build all N rows)."""
    seed = wl.seed + layer
    rows = [host_bf16((wl.hidden,), seed, TAG_X, 0, SIGMA_X, first=int(t) * wl.hidden) for t in tokens]
    x = np.stack(rows) if rows else np.empty((0, wl.hidden), np.uint16)
    if wl.zipf_s > 0 and len(x):
        x[:, 0] = 0x3F80
    return x


def host_expert(wl: Workload, e: int, layer: int = 0):
    """Routed expert ``e``: bf16 -> (Wg [I,H], Wu [I,H], Wd [H,I]) bit arrays;
    fp8 -> ((qg, sg), (qu, su), (qd, sd)) with per-128x128-block fp32 scales."""
    seed = wl.seed + layer
    I, H = wl.inter, wl.hidden
    if wl.weight_dtype == "bf16":
        return (host_bf16((I, H), seed, TAG_GATE, e, SIGMA_W), host_bf16((I, H), seed, TAG_UP, e, SIGMA_W),
                host_bf16((H, I), seed, TAG_DOWN, e, SIGMA_W))
    q = host_mxfp4 if wl.weight_dtype == "mxfp4" else host_e4m3
    return (q(I, H, seed, TAG_GATE, e, SIGMA_W), q(I, H, seed, TAG_UP, e, SIGMA_W), q(H, I, seed, TAG_DOWN, e, SIGMA_W))


def host_shared(wl: Workload, layer: int = 0):
    """The shared expert in the same form as ``host_expert``, or None."""
    if wl.shared_inter == 0:
        return None
    seed = wl.seed + layer
    Is, H = wl.shared_inter, wl.hidden
    if wl.weight_dtype == "bf16":
        return (host_bf16((Is, H), seed, TAG_SH_GATE, 0, SIGMA_W), host_bf16((Is, H), seed, TAG_SH_UP, 0, SIGMA_W),
                host_bf16((H, Is), seed, TAG_SH_DOWN, 0, SIGMA_W))
    q = host_mxfp4 if wl.weight_dtype == "mxfp4" else host_e4m3
    return (q(Is, H, seed, TAG_SH_GATE, 0, SIGMA_W), q(Is, H, seed, TAG_SH_UP, 0, SIGMA_W),
            q(H, Is, seed, TAG_SH_DOWN, 0, SIGMA_W))


def host_shared_gate(wl: Workload, layer: int = 0) -> Optional[np.ndarray]:
    """The shared expert's gate row [H] (bf16 bits, N(0, SIGMA_W)), or None."""
    if wl.shared_inter == 0 or not wl.shared_gated:
        return None
    return host_bf16((wl.hidden,), wl.seed + layer, TAG_SH_EXPERT_GATE, 0, SIGMA_W)


# ----------------------------------------------------------------------------- device fills (torch)

def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what}: HIP error {rc}")


def dev_bf16(t, seed: int, tag: int, sub: int, sigma: float, stream=None, first: int = 0) -> None:
    """Fill a contiguous torch bf16/int16 CUDA tensor in place."""
    import torch
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(_dev_lib().mi_dev_fill_bf16(t.data_ptr(), t.numel(), first, seed, tag, sub, sigma, s), "fill_bf16")


def dev_f32(t, seed: int, tag: int, sub: int, sigma: float, stream=None, first: int = 0) -> None:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(_dev_lib().mi_dev_fill_f32(t.data_ptr(), t.numel(), first, seed, tag, sub, sigma, s), "fill_f32")


def dev_mxfp4(q, scales, rows: int, cols: int, seed: int, tag: int, sub: int, sigma: float, stream=None) -> None:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(_dev_lib().mi_dev_fill_mxfp4(q.data_ptr(), scales.data_ptr(), rows, cols, seed, tag, sub, sigma, s),
           "fill_mxfp4")


def dev_e4m3(q, scales, rows: int, cols: int, seed: int, tag: int, sub: int, sigma: float, stream=None) -> None:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(_dev_lib().mi_dev_fill_e4m3(q.data_ptr(), scales.data_ptr(), rows, cols, seed, tag, sub, sigma, s),
           "fill_e4m3")
