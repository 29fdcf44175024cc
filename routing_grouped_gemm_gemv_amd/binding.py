"""ctypes binding of libmoe.so: the C ABI of include/moe.h, entry point for entry point.

Argument marshalling only.  Every function takes torch tensors that already
live on the current HIP device, checks their dtype, size and contiguity
against the layer shape, and passes raw pointers plus the current torch
stream to the library.  Every step of the layer runs in the library's HIP
kernels; there is no other implementation behind these names, and loading
fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB names another build of the same library (the sanitized host-only
# build the CPU tests load); by default the in-tree libmoe.so
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_BF16, MOE_F32 = 0, 1
MOE_SOFTMAX, MOE_SIGMOID, MOE_SQRTSOFTPLUS = 0, 1, 2
MOE_COMBINE_F32_FOLD, MOE_COMBINE_F64 = 0, 1

EXPORTED = (
    "moe_workspace_size",
    "moe_route",
    "moe_permute",
    "moe_experts",
    "moe_combine",
    "moe_forward",
    "moe_forward_noalloc",
    "moe_route_replay",
    "moe_forward_replay",
    "moe_backward_workspace_size",
    "moe_backward",
    "moe_status_string",
    "moe_last_error",
)


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str, message: str):
        super().__init__(f"{fn}: status {status}: {message}")
        self.status = status


class _Shape(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("D", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("I", ctypes.c_int32),
        ("Is", ctypes.c_int32),
        ("score", ctypes.c_int32),
        ("renorm", ctypes.c_int32),
        ("route_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("combine", ctypes.c_int32),
        ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
    ]


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("router", "gate_up", "down", "gate_up_shared", "down_shared")]


class _Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dx", "d_router", "d_gate_up", "d_down", "d_gate_up_shared",
                                                  "d_down_shared")]


class _Trace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("logits", "topk_ids", "topk_w", "counts", "offsets",
                                                  "perm_token", "inv_pos", "y", "shared_out")]


@dataclass(frozen=True)
class Shape:
    """The layer profile (moe_shape)."""
    T: int
    D: int
    E: int
    K: int
    I: int
    Is: int = 0
    score: str = "softmax"      # "softmax" | "sigmoid" | "sqrtsoftplus"
    renorm: bool = True
    route_scale: float = 1.0
    dtype: str = "bf16"         # operand dtype: "bf16" | "f32"
    combine: str = "f32"        # combine arithmetic: "f32" (float32 fold) | "f64" (order-invariant sum)
    n_group: int = 1            # group-limited select: expert groups (0 or 1: none)
    topk_group: int = 1         # groups kept per token

    def c(self) -> _Shape:
        return _Shape(self.T, self.D, self.E, self.K, self.I, self.Is,
                      {"softmax": MOE_SOFTMAX, "sigmoid": MOE_SIGMOID,
                       "sqrtsoftplus": MOE_SQRTSOFTPLUS}.get(self.score, -1),
                      int(self.renorm), float(self.route_scale),
                      {"bf16": MOE_BF16, "f32": MOE_F32}.get(self.dtype, -1),
                      {"f32": MOE_COMBINE_F32_FOLD, "f64": MOE_COMBINE_F64}.get(self.combine, -1),
                      int(self.n_group), int(self.topk_group))

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def replace(self, **kw) -> "Shape":
        d = dict(self.__dict__)
        d.update(kw)
        return Shape(**d)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with routing_grouped_gemm_gemv_amd.build.build()")
    # torch is imported first so that its HIP runtime is the one libmoe.so binds to
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    S = ctypes.POINTER(_Shape)
    L.moe_workspace_size.argtypes = [S, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_route.argtypes = [S, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_permute.argtypes = [S, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_experts.argtypes = [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_combine.argtypes = [S, P, P, P, P, ctypes.c_int32, P, P]
    L.moe_forward.argtypes = [S, ctypes.POINTER(_Weights), P, P, P, ctypes.c_int32, P,
                              ctypes.POINTER(_Trace), P, ctypes.c_size_t, P]
    L.moe_forward_noalloc.argtypes = [S, ctypes.POINTER(_Weights), P, P, P, ctypes.c_int32, P,
                                      ctypes.POINTER(_Trace), P]
    L.moe_route_replay.argtypes = [S, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_forward_replay.argtypes = [S, ctypes.POINTER(_Weights), P, P, P, ctypes.c_int32, P,
                                     ctypes.POINTER(_Trace), P, ctypes.c_size_t, P]
    L.moe_backward_workspace_size.argtypes = [S, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_backward.argtypes = [S, ctypes.POINTER(_Weights), P, P, ctypes.POINTER(_Trace), P,
                               ctypes.POINTER(_Grads), P, ctypes.c_size_t, P]
    for fn in ("moe_workspace_size", "moe_route", "moe_permute", "moe_experts", "moe_combine", "moe_forward",
               "moe_forward_noalloc", "moe_route_replay", "moe_forward_replay", "moe_backward_workspace_size", "moe_backward"):
        getattr(L, fn).restype = ctypes.c_int
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int, fn: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, fn, lib().moe_last_error().decode())


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, numel=None) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def workspace_size(shape: Shape) -> int:
    n = ctypes.c_size_t(0)
    s = shape.c()
    _check(lib().moe_workspace_size(ctypes.byref(s), ctypes.byref(n)), "moe_workspace_size")
    return int(n.value)


def alloc_workspace(shape: Shape, device=None) -> torch.Tensor:
    return torch.empty(max(workspace_size(shape), 1), dtype=torch.uint8, device=device or "cuda")


def moe_route(shape: Shape, x, router, sel_bias, mask, logits, topk_ids, topk_w, ws) -> None:
    s = shape.c()
    od = shape.torch_dtype
    _check(lib().moe_route(
        ctypes.byref(s),
        _ptr(x, "x", od, shape.T * shape.D), _ptr(router, "router", od, shape.E * shape.D),
        _ptr(sel_bias, "sel_bias", torch.float32, shape.E), _ptr(mask, "mask", torch.uint8, shape.T),
        _ptr(logits, "logits", torch.float32, shape.T * shape.E),
        _ptr(topk_ids, "topk_ids", torch.int32, shape.T * shape.K),
        _ptr(topk_w, "topk_w", torch.float32, shape.T * shape.K),
        _ptr(ws, "ws", torch.uint8), ws.numel() if ws is not None else 0, _stream()), "moe_route")


def moe_route_replay(shape: Shape, x, router, replay_ids, mask, logits, topk_ids, topk_w, ws) -> None:
    s = shape.c()
    od = shape.torch_dtype
    _check(lib().moe_route_replay(
        ctypes.byref(s),
        _ptr(x, "x", od, shape.T * shape.D), _ptr(router, "router", od, shape.E * shape.D),
        _ptr(replay_ids, "replay_ids", torch.int32, shape.T * shape.K), _ptr(mask, "mask", torch.uint8, shape.T),
        _ptr(logits, "logits", torch.float32, shape.T * shape.E),
        _ptr(topk_ids, "topk_ids", torch.int32, shape.T * shape.K),
        _ptr(topk_w, "topk_w", torch.float32, shape.T * shape.K),
        _ptr(ws, "ws", torch.uint8), ws.numel() if ws is not None else 0, _stream()), "moe_route_replay")


def moe_permute(shape: Shape, topk_ids, counts, offsets, perm_token, inv_pos, ws) -> None:
    s = shape.c()
    P = shape.T * shape.K
    _check(lib().moe_permute(
        ctypes.byref(s), _ptr(topk_ids, "topk_ids", torch.int32, P),
        _ptr(counts, "counts", torch.int32, shape.E), _ptr(offsets, "offsets", torch.int32, shape.E + 1),
        _ptr(perm_token, "perm_token", torch.int32, P), _ptr(inv_pos, "inv_pos", torch.int32, P),
        _ptr(ws, "ws", torch.uint8), ws.numel() if ws is not None else 0, _stream()), "moe_permute")


def moe_experts(shape: Shape, x, perm_token, offsets, gate_up, down, y, ws) -> None:
    s = shape.c()
    od = shape.torch_dtype
    _check(lib().moe_experts(
        ctypes.byref(s), _ptr(x, "x", od), _ptr(perm_token, "perm_token", torch.int32),
        _ptr(offsets, "offsets", torch.int32, shape.E + 1),
        _ptr(gate_up, "gate_up", od, shape.E * 2 * shape.I * shape.D),
        _ptr(down, "down", od, shape.E * shape.D * shape.I),
        _ptr(y, "y", od), _ptr(ws, "ws", torch.uint8), ws.numel() if ws is not None else 0,
        _stream()), "moe_experts")


def moe_combine(shape: Shape, y, inv_pos, topk_w, shared_out, out) -> None:
    s = shape.c()
    od = shape.torch_dtype
    out_dtype = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}[out.dtype]
    _check(lib().moe_combine(
        ctypes.byref(s), _ptr(y, "y", od), _ptr(inv_pos, "inv_pos", torch.int32, shape.T * shape.K),
        _ptr(topk_w, "topk_w", torch.float32, shape.T * shape.K),
        _ptr(shared_out, "shared_out", od, shape.T * shape.D),
        out_dtype, _ptr(out, "out", None, shape.T * shape.D), _stream()), "moe_combine")


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def moe_forward_noalloc(shape: Shape, weights: dict, x, sel_bias, mask, out, trace: Optional[dict] = None) -> None:
    """moe_forward on the library's fixed device scratch (no workspace argument)."""
    _forward_call(shape, weights, x, sel_bias, mask, out, None, trace, None, noalloc=True)


def moe_forward(shape: Shape, weights: dict, x, sel_bias, mask, out, ws, trace: Optional[dict] = None,
                replay_ids=None) -> None:
    """weights: router, gate_up, down[, gate_up_shared, down_shared]; trace: optional
    dict of preallocated boundary tensors keyed like moe_trace's fields.  With
    ``replay_ids`` ([T, K] int32) this calls moe_forward_replay instead."""
    _forward_call(shape, weights, x, sel_bias, mask, out, ws, trace, replay_ids)


def _forward_call(shape: Shape, weights: dict, x, sel_bias, mask, out, ws, trace, replay_ids,
                  noalloc: bool = False) -> None:
    s = shape.c()
    od = shape.torch_dtype
    w = _Weights(
        _ptr(weights["router"], "router", od, shape.E * shape.D),
        _ptr(weights["gate_up"], "gate_up", od, shape.E * 2 * shape.I * shape.D),
        _ptr(weights["down"], "down", od, shape.E * shape.D * shape.I),
        _ptr(weights.get("gate_up_shared"), "gate_up_shared", od, 2 * shape.Is * shape.D),
        _ptr(weights.get("down_shared"), "down_shared", od, shape.D * shape.Is),
    )
    tr = None
    if trace:
        P = shape.T * shape.K
        tr = _Trace(
            _ptr(trace.get("logits"), "logits", torch.float32, shape.T * shape.E),
            _ptr(trace.get("topk_ids"), "topk_ids", torch.int32, P),
            _ptr(trace.get("topk_w"), "topk_w", torch.float32, P),
            _ptr(trace.get("counts"), "counts", torch.int32, shape.E),
            _ptr(trace.get("offsets"), "offsets", torch.int32, shape.E + 1),
            _ptr(trace.get("perm_token"), "perm_token", torch.int32, P),
            _ptr(trace.get("inv_pos"), "inv_pos", torch.int32, P),
            _ptr(trace.get("y"), "y", od, P * shape.D),
            _ptr(trace.get("shared_out"), "shared_out", od, shape.T * shape.D),
        )
    out_dtype = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}[out.dtype]
    if replay_ids is not None:
        _check(lib().moe_forward_replay(
            ctypes.byref(s), ctypes.byref(w), _ptr(x, "x", od, shape.T * shape.D),
            _ptr(replay_ids, "replay_ids", torch.int32, shape.T * shape.K), _ptr(mask, "mask", torch.uint8, shape.T),
            out_dtype, _ptr(out, "out", None, shape.T * shape.D),
            ctypes.byref(tr) if tr is not None else None,
            _ptr(ws, "ws", torch.uint8), ws.numel() if ws is not None else 0, _stream()), "moe_forward_replay")
        return
    if noalloc:
        _check(lib().moe_forward_noalloc(
            ctypes.byref(s), ctypes.byref(w), _ptr(x, "x", od, shape.T * shape.D),
            _ptr(sel_bias, "sel_bias", torch.float32, shape.E), _ptr(mask, "mask", torch.uint8, shape.T),
            out_dtype, _ptr(out, "out", None, shape.T * shape.D),
            ctypes.byref(tr) if tr is not None else None, _stream()), "moe_forward_noalloc")
        return
    _check(lib().moe_forward(
        ctypes.byref(s), ctypes.byref(w), _ptr(x, "x", od, shape.T * shape.D),
        _ptr(sel_bias, "sel_bias", torch.float32, shape.E), _ptr(mask, "mask", torch.uint8, shape.T),
        out_dtype, _ptr(out, "out", None, shape.T * shape.D),
        ctypes.byref(tr) if tr is not None else None,
        _ptr(ws, "ws", torch.uint8), ws.numel() if ws is not None else 0, _stream()), "moe_forward")


def backward_workspace_size(shape: Shape) -> int:
    n = ctypes.c_size_t(0)
    s = shape.c()
    _check(lib().moe_backward_workspace_size(ctypes.byref(s), ctypes.byref(n)), "moe_backward_workspace_size")
    return int(n.value)


def moe_backward(shape: Shape, weights: dict, x, mask, trace: dict, dout, grads: dict, ws) -> None:
    """Gradients of the layer (moe_backward).  trace: the forward's boundary
    tensors (topk_ids, topk_w, offsets, perm_token, inv_pos, y); grads: float32
    tensors dx, d_router, d_gate_up, d_down[, d_gate_up_shared, d_down_shared]."""
    s = shape.c()
    od = shape.torch_dtype
    P = shape.T * shape.K
    f32 = torch.float32
    w = _Weights(
        _ptr(weights["router"], "router", od, shape.E * shape.D),
        _ptr(weights["gate_up"], "gate_up", od, shape.E * 2 * shape.I * shape.D),
        _ptr(weights["down"], "down", od, shape.E * shape.D * shape.I),
        _ptr(weights.get("gate_up_shared"), "gate_up_shared", od, 2 * shape.Is * shape.D),
        _ptr(weights.get("down_shared"), "down_shared", od, shape.D * shape.Is),
    )
    tr = _Trace(
        None,
        _ptr(trace["topk_ids"], "topk_ids", torch.int32, P),
        _ptr(trace["topk_w"], "topk_w", f32, P),
        None,
        _ptr(trace["offsets"], "offsets", torch.int32, shape.E + 1),
        _ptr(trace["perm_token"], "perm_token", torch.int32, P),
        _ptr(trace["inv_pos"], "inv_pos", torch.int32, P),
        _ptr(trace["y"], "y", od, P * shape.D),
        None,
    )
    g = _Grads(
        _ptr(grads["dx"], "dx", f32, shape.T * shape.D),
        _ptr(grads["d_router"], "d_router", f32, shape.E * shape.D),
        _ptr(grads["d_gate_up"], "d_gate_up", f32, shape.E * 2 * shape.I * shape.D),
        _ptr(grads["d_down"], "d_down", f32, shape.E * shape.D * shape.I),
        _ptr(grads.get("d_gate_up_shared"), "d_gate_up_shared", f32, 2 * shape.Is * shape.D),
        _ptr(grads.get("d_down_shared"), "d_down_shared", f32, shape.D * shape.Is),
    )
    _check(lib().moe_backward(
        ctypes.byref(s), ctypes.byref(w), _ptr(x, "x", od, shape.T * shape.D), _ptr(mask, "mask", torch.uint8, shape.T),
        ctypes.byref(tr), _ptr(dout, "dout", od, shape.T * shape.D), ctypes.byref(g),
        _ptr(ws, "ws", torch.uint8), ws.numel() if ws is not None else 0, _stream()), "moe_backward")
