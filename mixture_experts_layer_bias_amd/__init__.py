"""Python binding of libmoe, the gfx950 MoE layer forward (C ABI in include/moe.h).

Argument marshalling only: every function passes torch tensors' device
pointers and the current HIP stream to the function of the same name in
libmoe.so, and raises ``MoeError`` with the library's message when it returns
a failure status.  Nothing here computes any part of the layer, and nothing
falls back to another implementation: if libmoe.so is missing, every call
raises.

bf16 tensors are ``torch.bfloat16``; e4m3 tensors are ``torch.uint8`` or
``torch.float8_e4m3fn``; ids are ``torch.int32``; weights and scales of the
routing are ``torch.float32``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, 1, 2, 3, 4
MOE_SCORING_SOFTMAX, MOE_SCORING_SIGMOID, MOE_SCORING_SQRTSOFTPLUS = 0, 1, 2
MOE_WEIGHTS_BF16, MOE_WEIGHTS_FP8_E4M3, MOE_WEIGHTS_MXFP4 = 0, 1, 2
MOE_STAGE_GATE_UP, MOE_STAGE_DOWN = 0, 1
MOE_GROUP_ROUTED, MOE_GROUP_SHARED = 0, 1

EXPORTED = ["moe_workspace_size", "moe_workspace_layout", "moe_route_topk", "moe_permute", "moe_quantize_fp8",
            "moe_grouped_gemm", "moe_unpermute_reduce", "moe_forward", "moe_experts_forward", "moe_forward_noalloc",
            "moe_status_str", "moe_last_error"]
MOE_NOALLOC_WORKSPACE_BYTES = 32 << 20  # the static workspace of moe_forward_noalloc


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status
        self.message = message


class moe_config_t(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("router_width", ctypes.c_int32), ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("scoring", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("weight_dtype", ctypes.c_int32), ("row_invariant", ctypes.c_int32)]


class moe_weights_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router_w", "correction_bias", "gate_w", "up_w", "down_w", "gate_s", "up_s", "down_s",
        "sh_gate_w", "sh_up_w", "sh_down_w", "sh_gate_s", "sh_up_s", "sh_down_s", "sh_expert_gate")]


class moe_workspace_layout_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "logits", "topk_ids", "topk_w", "zero_w", "counts", "offsets", "sorted_ids", "inv_perm", "xq", "x_scales",
        "h", "h_scales", "y", "shared_h", "shared_h_scales", "shared_y", "scratch", "sync", "sync_error", "split",
        "total")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run mixture_experts_layer_bias_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        cfgp = ctypes.POINTER(moe_config_t)
        sig = {
            "moe_workspace_size": [cfgp, ctypes.POINTER(sz)],
            "moe_workspace_layout": [cfgp, ctypes.POINTER(moe_workspace_layout_t)],
            "moe_route_topk": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_permute": [cfgp, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_quantize_fp8": [cfgp, vp, vp, vp, vp],
            "moe_grouped_gemm": [cfgp, i32, i32, ctypes.POINTER(moe_weights_t), vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_unpermute_reduce": [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "moe_forward": [cfgp, ctypes.POINTER(moe_weights_t), vp, vp, vp, sz, vp],
            "moe_experts_forward": [cfgp, ctypes.POINTER(moe_weights_t), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "moe_forward_noalloc": [cfgp, ctypes.POINTER(moe_weights_t), vp, vp, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _status_name(status: int) -> str:
    try:
        return lib().moe_status_str(status).decode()
    except Exception:  # noqa: BLE001 - naming only
        return f"status {status}"


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


# ----------------------------------------------------------------------------- config

def make_config(num_tokens: int, hidden: int, num_experts: int, router_width: int, top_k: int, inter: int,
                shared_inter: int = 0, scoring: str = "softmax", renormalize: bool = True,
                routed_scale: float = 1.0, weight_dtype: str = "bf16", row_invariant: bool = False) -> moe_config_t:
    return moe_config_t(num_tokens, hidden, num_experts, router_width, top_k, inter, shared_inter,
                        {"softmax": MOE_SCORING_SOFTMAX, "sigmoid": MOE_SCORING_SIGMOID,
                         "sqrtsoftplus": MOE_SCORING_SQRTSOFTPLUS}[scoring],
                        1 if renormalize else 0, routed_scale,
                        {"bf16": MOE_WEIGHTS_BF16, "fp8": MOE_WEIGHTS_FP8_E4M3, "mxfp4": MOE_WEIGHTS_MXFP4}[weight_dtype],
                        1 if row_invariant else 0)


def config_with_tokens(cfg: moe_config_t, n: int) -> moe_config_t:
    c = moe_config_t.from_buffer_copy(cfg)
    c.num_tokens = n
    return c


# ----------------------------------------------------------------------------- marshalling

def _ptr(t, name: str, elem_size: Optional[int] = None, optional: bool = False) -> Optional[int]:
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if isinstance(t, int):  # a raw device address
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if elem_size is not None and t.element_size() != elem_size:
        raise ValueError(f"{name} has element size {t.element_size()}, expected {elem_size}")
    return t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclasses.dataclass
class LayerWeights:
    """Device weights of one layer, plus the per-expert pointer tables that
    libmoe reads.  Holds references to every tensor so the pointers stay valid."""

    router_w: object  # [R, H] bf16
    correction_bias: Optional[object]  # [R] f32
    gate_w: Sequence  # E tensors [I, H]
    up_w: Sequence
    down_w: Sequence  # E tensors [H, I]
    gate_s: Optional[Sequence] = None  # fp8: E tensors [I/128, H/128] f32
    up_s: Optional[Sequence] = None
    down_s: Optional[Sequence] = None
    sh_gate_w: Optional[object] = None
    sh_up_w: Optional[object] = None
    sh_down_w: Optional[object] = None
    sh_gate_s: Optional[object] = None
    sh_up_s: Optional[object] = None
    sh_down_s: Optional[object] = None
    sh_expert_gate: Optional[object] = None  # [H] bf16: the shared expert's sigmoid gate row

    def __post_init__(self):
        import torch
        dev = self.router_w.device

        def table(ts):
            if ts is None:
                return None
            return torch.tensor([_ptr(t, "expert weight") for t in ts], dtype=torch.int64, device=dev)

        self._tables = {n: table(getattr(self, n)) for n in ("gate_w", "up_w", "down_w", "gate_s", "up_s",
                                                             "down_s")}
        s = moe_weights_t()
        s.router_w = _ptr(self.router_w, "router_w", 2)
        s.correction_bias = _ptr(self.correction_bias, "correction_bias", 4, optional=True)
        for n, t in self._tables.items():
            setattr(s, n, None if t is None else t.data_ptr())
        for n in ("sh_gate_w", "sh_up_w", "sh_down_w", "sh_gate_s", "sh_up_s", "sh_down_s", "sh_expert_gate"):
            setattr(s, n, _ptr(getattr(self, n), n, optional=True))
        self.struct = s


def moe_workspace_size(cfg: moe_config_t) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def moe_workspace_layout(cfg: moe_config_t) -> dict:
    L = moe_workspace_layout_t()
    _check(lib().moe_workspace_layout(ctypes.byref(cfg), ctypes.byref(L)))
    return {name: getattr(L, name) for name, _ in moe_workspace_layout_t._fields_}


def moe_route_topk(cfg, x, router_w, correction_bias, logits, topk_ids, topk_w, zero_w, ws, stream=None) -> None:
    _check(lib().moe_route_topk(ctypes.byref(cfg), _ptr(x, "x", 2), _ptr(router_w, "router_w", 2),
                                _ptr(correction_bias, "correction_bias", 4, True), _ptr(logits, "logits", 4),
                                _ptr(topk_ids, "topk_ids", 4), _ptr(topk_w, "topk_w", 4),
                                _ptr(zero_w, "zero_w", 4, True), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
                                _stream(stream)))


def moe_permute(cfg, topk_ids, counts, offsets, sorted_ids, inv_perm, ws, stream=None) -> None:
    _check(lib().moe_permute(ctypes.byref(cfg), _ptr(topk_ids, "topk_ids", 4), _ptr(counts, "counts", 4),
                             _ptr(offsets, "offsets", 4), _ptr(sorted_ids, "sorted_ids", 4),
                             _ptr(inv_perm, "inv_perm", 4), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
                             _stream(stream)))


def moe_quantize_fp8(cfg, x, xq, x_scales, stream=None) -> None:
    _check(lib().moe_quantize_fp8(ctypes.byref(cfg), _ptr(x, "x", 2), _ptr(xq, "xq", 1),
                                  _ptr(x_scales, "x_scales", 4), _stream(stream)))


def moe_grouped_gemm(cfg, stage: int, group: int, weights: LayerWeights, a, a_scales, sorted_ids, offsets, out,
                     out_scales=None, ws=None, stream=None) -> None:
    _check(lib().moe_grouped_gemm(ctypes.byref(cfg), stage, group, ctypes.byref(weights.struct), _ptr(a, "a"),
                                  _ptr(a_scales, "a_scales", 4, True), _ptr(sorted_ids, "sorted_ids", 4, True),
                                  _ptr(offsets, "offsets", 4, True), _ptr(out, "out"),
                                  _ptr(out_scales, "out_scales", 4, True), _ptr(ws, "ws", optional=True),
                                  0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_unpermute_reduce(cfg, y_sorted, inv_perm, topk_ids, topk_w, x, shared_y, out, shared_gate=None,
                         stream=None) -> None:
    _check(lib().moe_unpermute_reduce(ctypes.byref(cfg), _ptr(y_sorted, "y_sorted", 2), _ptr(inv_perm, "inv_perm", 4),
                                      _ptr(topk_ids, "topk_ids", 4), _ptr(topk_w, "topk_w", 4), _ptr(x, "x", 2),
                                      _ptr(shared_y, "shared_y", 2, True), _ptr(shared_gate, "shared_gate", 2, True),
                                      _ptr(out, "out", 2), _stream(stream)))


def moe_forward(cfg, weights: LayerWeights, x, out, ws, stream=None) -> None:
    _check(lib().moe_forward(ctypes.byref(cfg), ctypes.byref(weights.struct), _ptr(x, "x", 2), _ptr(out, "out", 2),
                             _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)))


def moe_forward_noalloc(cfg, weights: LayerWeights, x, out, stream=None) -> None:
    _check(lib().moe_forward_noalloc(ctypes.byref(cfg), ctypes.byref(weights.struct), _ptr(x, "x", 2),
                                     _ptr(out, "out", 2), _stream(stream)))


def moe_experts_forward(cfg, weights: LayerWeights, x, topk_ids, topk_w, offsets, sorted_ids, inv_perm, out, ws,
                        stream=None) -> None:
    _check(lib().moe_experts_forward(ctypes.byref(cfg), ctypes.byref(weights.struct), _ptr(x, "x", 2),
                                     _ptr(topk_ids, "topk_ids", 4), _ptr(topk_w, "topk_w", 4),
                                     _ptr(offsets, "offsets", 4), _ptr(sorted_ids, "sorted_ids", 4),
                                     _ptr(inv_perm, "inv_perm", 4), _ptr(out, "out", 2), _ptr(ws, "ws"),
                                     ws.numel() * ws.element_size(), _stream(stream)))


def weights_from_stacked(router_w, correction_bias, gate, up, down, gate_s=None, up_s=None, down_s=None,
                         sh_gate=None, sh_up=None, sh_down=None, sh_gate_s=None, sh_up_s=None,
                         sh_down_s=None, sh_expert_gate=None) -> LayerWeights:
    """LayerWeights over expert weights stacked as [E, I, H] / [E, H, I] tensors
    (and [E, ., .] block scales for fp8): the tables point at each expert's slice."""
    E = gate.shape[0]

    def split(t):
        return None if t is None else [t[e] for e in range(E)]

    return LayerWeights(router_w, correction_bias, split(gate), split(up), split(down), split(gate_s), split(up_s),
                        split(down_s), sh_gate, sh_up, sh_down, sh_gate_s, sh_up_s, sh_down_s, sh_expert_gate)
