"""The C ABI on the CPU: the library loads, exports every declared entry point,
and rejects bad arguments before it touches a device (no compute calls)."""

import ctypes
import os
import re
import subprocess

import pytest

import routing_grouped_gemm_gemv_amd as moe
from routing_grouped_gemm_gemv_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)$", out, re.M))
    assert set(declared_functions()) <= exported


def _shape(**kw):
    base = dict(T=64, D=128, E=8, K=2, I=256, Is=0, score=0, renorm=1, route_scale=1.0, dtype=0, combine=0,
                n_group=0, topk_group=0)
    base.update(kw)
    return B._Shape(base["T"], base["D"], base["E"], base["K"], base["I"], base["Is"], base["score"],
                    base["renorm"], base["route_scale"], base["dtype"], base["combine"], base["n_group"],
                    base["topk_group"])


@pytest.mark.parametrize("kw,status", [
    (dict(), B.MOE_OK),
    (dict(T=-1), B.MOE_ERR_INVALID),
    (dict(D=0), B.MOE_ERR_INVALID),
    (dict(K=9), B.MOE_ERR_INVALID),
    (dict(score=2), B.MOE_OK),
    (dict(score=3), B.MOE_ERR_INVALID),
    (dict(n_group=1, topk_group=0), B.MOE_OK),
    (dict(n_group=4, topk_group=2), B.MOE_OK),
    (dict(n_group=4, topk_group=2, K=5), B.MOE_ERR_INVALID),
    (dict(n_group=4, topk_group=0), B.MOE_ERR_INVALID),
    (dict(n_group=4, topk_group=5), B.MOE_ERR_INVALID),
    (dict(n_group=3, topk_group=1), B.MOE_ERR_INVALID),
    (dict(n_group=8, topk_group=2), B.MOE_ERR_INVALID),
    (dict(n_group=-1), B.MOE_ERR_INVALID),
    (dict(E=256, n_group=128, topk_group=4), B.MOE_ERR_UNSUPPORTED),
    (dict(dtype=3), B.MOE_ERR_INVALID),
    (dict(renorm=2), B.MOE_ERR_INVALID),
    (dict(combine=2), B.MOE_ERR_INVALID),
    (dict(combine=1), B.MOE_OK),
    (dict(route_scale=0.0), B.MOE_ERR_INVALID),
    (dict(route_scale=float("nan")), B.MOE_ERR_INVALID),
    (dict(route_scale=float("inf")), B.MOE_ERR_INVALID),
    (dict(D=100), B.MOE_ERR_UNSUPPORTED),
    (dict(I=96), B.MOE_ERR_UNSUPPORTED),
    (dict(Is=32), B.MOE_ERR_UNSUPPORTED),
    (dict(E=2048, K=2), B.MOE_ERR_UNSUPPORTED),
    (dict(E=64, K=17), B.MOE_ERR_UNSUPPORTED),
    (dict(T=2 ** 30, K=2), B.MOE_ERR_UNSUPPORTED),
])
def test_shape_validation(kw, status):
    L = moe.lib()
    s = _shape(**kw)
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == status
    if status != B.MOE_OK:
        assert L.moe_last_error().decode() != ""
        assert L.moe_status_string(status).decode().startswith("MOE_ERR")
    else:
        assert n.value > 0


def test_null_shape_and_pointers_are_rejected_before_any_launch():
    L = moe.lib()
    s = _shape()
    one = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    assert L.moe_workspace_size(None, None) == B.MOE_ERR_INVALID
    assert L.moe_route(None, one, one, None, None, None, one, one, one, 1 << 30, None) == B.MOE_ERR_INVALID
    assert L.moe_route(ctypes.byref(s), None, one, None, None, None, one, one, one, 1 << 30, None) == B.MOE_ERR_INVALID
    assert L.moe_permute(ctypes.byref(s), one, None, one, one, one, one, 1 << 30, None) == B.MOE_ERR_INVALID
    assert L.moe_experts(ctypes.byref(s), one, one, None, one, one, one, one, 1 << 30, None) == B.MOE_ERR_INVALID
    assert L.moe_combine(ctypes.byref(s), one, one, one, None, 7, one, None) == B.MOE_ERR_INVALID
    w = B._Weights(16, None, 16, None, None)
    assert L.moe_forward(ctypes.byref(s), ctypes.byref(w), one, None, None, 0, one, None, one, 1 << 30, None) \
        == B.MOE_ERR_INVALID
    s2 = _shape(Is=64)
    w2 = B._Weights(16, 16, 16, None, None)
    assert L.moe_forward(ctypes.byref(s2), ctypes.byref(w2), one, None, None, 0, one, None, one, 1 << 30, None) \
        == B.MOE_ERR_INVALID
    assert "Is > 0" in L.moe_last_error().decode()


def test_small_workspace_is_rejected_before_any_launch():
    L = moe.lib()
    s = _shape()
    one = ctypes.c_void_p(16)
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == B.MOE_OK
    w = B._Weights(16, 16, 16, None, None)
    assert L.moe_forward(ctypes.byref(s), ctypes.byref(w), one, None, None, 0, one, None, one, n.value - 1, None) \
        == B.MOE_ERR_WORKSPACE
    assert L.moe_forward(ctypes.byref(s), ctypes.byref(w), one, None, None, 0, one, None, None, n.value, None) \
        == B.MOE_ERR_WORKSPACE
    assert L.moe_route(ctypes.byref(s), one, one, None, None, None, one, one, one, 8, None) == B.MOE_ERR_WORKSPACE
    assert L.moe_permute(ctypes.byref(s), one, one, one, one, one, one, 0, None) == B.MOE_ERR_WORKSPACE
    assert L.moe_experts(ctypes.byref(s), one, one, one, one, one, one, one, 0, None) == B.MOE_ERR_WORKSPACE


def test_zero_tokens_launch_nothing():
    L = moe.lib()
    s = _shape(T=0)
    one = ctypes.c_void_p(16)
    w = B._Weights(16, 16, 16, None, None)
    assert L.moe_route(ctypes.byref(s), one, one, None, None, None, one, one, None, 0, None) == B.MOE_OK
    assert L.moe_permute(ctypes.byref(s), one, one, one, one, one, None, 0, None) == B.MOE_OK
    assert L.moe_experts(ctypes.byref(s), one, one, one, one, one, one, None, 0, None) == B.MOE_OK
    assert L.moe_combine(ctypes.byref(s), one, one, one, None, 0, one, None) == B.MOE_OK
    assert L.moe_forward(ctypes.byref(s), ctypes.byref(w), one, None, None, 0, one, None, None, 0, None) == B.MOE_OK


def test_workspace_grows_with_tokens_and_shared_expert():
    a = B.workspace_size(B.Shape(T=256, D=2048, E=128, K=8, I=768))
    b = B.workspace_size(B.Shape(T=512, D=2048, E=128, K=8, I=768))
    c = B.workspace_size(B.Shape(T=512, D=2048, E=128, K=8, I=768, Is=512))
    assert 0 < a < b < c
    # y alone: T*K rows of D bf16
    assert b >= 512 * 8 * 2048 * 2


def test_binding_rejects_host_tensors():
    import torch
    shape = B.Shape(T=4, D=128, E=8, K=2, I=256, dtype="f32")
    with pytest.raises(ValueError):
        B.moe_combine(shape, torch.zeros(8, 128), torch.zeros(4, 2, dtype=torch.int32),
                      torch.zeros(4, 2), None, torch.zeros(4, 128))


def test_backward_validation_before_launch():
    L = moe.lib()
    one = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    n = ctypes.c_size_t(0)
    s = _shape(dtype=0)
    assert L.moe_backward_workspace_size(ctypes.byref(s), ctypes.byref(n)) == B.MOE_OK and n.value > 0
    w = B._Weights(one, one, one, None, None)
    tr = B._Trace(None, one, one, None, one, one, one, one, None)
    g = B._Grads(one, one, one, one, None, None)
    # fp32 operands: not supported by the backward
    s32 = _shape(dtype=1)
    assert L.moe_backward(ctypes.byref(s32), ctypes.byref(w), one, None, ctypes.byref(tr), one, ctypes.byref(g),
                          one, 1 << 30, None) == B.MOE_ERR_UNSUPPORTED
    # a forward trace without y
    tr2 = B._Trace(None, one, one, None, one, one, one, None, None)
    assert L.moe_backward(ctypes.byref(s), ctypes.byref(w), one, None, ctypes.byref(tr2), one, ctypes.byref(g),
                          one, 1 << 30, None) == B.MOE_ERR_INVALID
    # a shared expert needs its gradient buffers
    s2 = _shape(Is=64)
    w2 = B._Weights(one, one, one, one, one)
    assert L.moe_backward(ctypes.byref(s2), ctypes.byref(w2), one, None, ctypes.byref(tr), one, ctypes.byref(g),
                          one, 1 << 30, None) == B.MOE_ERR_INVALID
    # too small a workspace
    assert L.moe_backward(ctypes.byref(s), ctypes.byref(w), one, None, ctypes.byref(tr), one, ctypes.byref(g),
                          one, 16, None) == B.MOE_ERR_WORKSPACE
    # a misaligned gradient buffer
    g2 = B._Grads(one, ctypes.c_void_p(20), one, one, None, None)
    assert L.moe_backward(ctypes.byref(s), ctypes.byref(w), one, None, ctypes.byref(tr), one, ctypes.byref(g2),
                          one, 1 << 30, None) == B.MOE_ERR_INVALID


def test_misaligned_pointers_are_rejected_before_launch():
    """Activations, weights, outputs and workspace move in 16-byte vectors,
    index arrays and per-token floats in 4-byte words: a pointer off that
    alignment is an argument error, found before anything is launched."""
    L = moe.lib()
    a16 = ctypes.c_void_p(256)
    odd8 = ctypes.c_void_p(264)   # 8-byte aligned only
    odd2 = ctypes.c_void_p(258)
    n = ctypes.c_size_t(1 << 30)
    s = _shape()
    INV = B.MOE_ERR_INVALID
    # route: x off 16 bytes; topk_ids off 4 bytes
    assert L.moe_route(ctypes.byref(s), odd8, a16, None, None, None, a16, a16, a16, n.value, None) == INV
    assert L.moe_route(ctypes.byref(s), a16, a16, None, None, None, odd2, a16, a16, n.value, None) == INV
    # permute: the workspace off 16 bytes
    assert L.moe_permute(ctypes.byref(s), a16, a16, a16, a16, a16, odd8, n.value, None) == INV
    # experts: y off 16 bytes
    assert L.moe_experts(ctypes.byref(s), a16, a16, a16, a16, a16, odd8, a16, n.value, None) == INV
    # combine: out off 16 bytes
    assert L.moe_combine(ctypes.byref(s), a16, a16, a16, None, 0, odd8, None) == INV
    # forward: a weight off 16 bytes; a trace array off 4 bytes (also with T = 0)
    w = B._Weights(a16, odd8, a16, None, None)
    assert L.moe_forward(ctypes.byref(s), ctypes.byref(w), a16, None, None, 0, a16, None, a16, n.value, None) == INV
    w = B._Weights(a16, a16, a16, None, None)
    tr = B._Trace(None, odd2, None, None, None, None, None, None, None)
    s0 = _shape(T=0)
    assert L.moe_forward(ctypes.byref(s0), ctypes.byref(w), a16, None, None, 0, a16, ctypes.byref(tr), a16,
                         n.value, None) == INV


def test_noalloc_forward_host_checks():
    """moe_forward_noalloc refuses shapes whose workspace exceeds its fixed
    scratch, and validates like moe_forward, before touching a device."""
    L = moe.lib()
    one = ctypes.c_void_p(16)
    w = B._Weights(16, 16, 16, None, None)
    big = _shape(T=8192, D=2048, E=128, K=8, I=768)
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(big), ctypes.byref(n)) == B.MOE_OK
    assert n.value > B.NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(ctypes.byref(big), ctypes.byref(w), one, None, None, 0, one, None, None) \
        == B.MOE_ERR_UNSUPPORTED
    assert "scratch" in L.moe_last_error().decode()
    s0 = _shape(T=0)
    assert L.moe_forward_noalloc(ctypes.byref(s0), ctypes.byref(w), one, None, None, 0, one, None, None) == B.MOE_OK
    wbad = B._Weights(16, None, 16, None, None)
    assert L.moe_forward_noalloc(ctypes.byref(_shape()), ctypes.byref(wbad), one, None, None, 0, one, None, None) \
        == B.MOE_ERR_INVALID
