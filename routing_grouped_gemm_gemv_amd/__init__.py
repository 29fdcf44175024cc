"""Sparse-MoE layer forward on one MI355X (gfx950): routing, dispatch, grouped
SwiGLU experts and a fixed-order combine, as hand-written HIP kernels behind
the C ABI of include/moe.h.  This package is the thin Python binding."""

from .binding import (
    EXPORTED,
    LIB_PATH,
    MOE_BF16,
    MOE_ERR_HIP,
    MOE_ERR_INVALID,
    MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE,
    MOE_F32,
    MOE_OK,
    MoeError,
    Shape,
    alloc_workspace,
    lib,
    moe_combine,
    moe_experts,
    moe_forward,
    moe_permute,
    moe_route,
    workspace_size,
)
from .layer import MoeLayer

__all__ = [
    "EXPORTED", "LIB_PATH", "MOE_BF16", "MOE_F32", "MOE_OK", "MOE_ERR_HIP", "MOE_ERR_INVALID",
    "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MoeError", "Shape", "alloc_workspace", "lib",
    "moe_combine", "moe_experts", "moe_forward", "moe_permute", "moe_route", "workspace_size",
    "MoeLayer",
]
