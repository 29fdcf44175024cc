"""A layer object holding device weights, over the C ABI (allocation and marshalling only)."""

from __future__ import annotations

from typing import Dict, Optional

import torch

from . import binding as B


class MoeLayer:
    """Device-resident weights of one MoE layer plus its shape.

    ``forward`` runs moe_forward; ``forward_stages`` runs moe_route,
    moe_permute, moe_experts (routed, then shared) and moe_combine one after
    another on the same stream and must give the same bits.
    """

    def __init__(self, shape: B.Shape, router: torch.Tensor, gate_up: torch.Tensor, down: torch.Tensor,
                 gate_up_shared: Optional[torch.Tensor] = None, down_shared: Optional[torch.Tensor] = None,
                 sel_bias: Optional[torch.Tensor] = None):
        self.shape = shape
        self.weights = {"router": router, "gate_up": gate_up, "down": down}
        if shape.Is > 0:
            self.weights["gate_up_shared"] = gate_up_shared
            self.weights["down_shared"] = down_shared
        self.sel_bias = sel_bias
        self._ws = None

    def with_tokens(self, T: int) -> B.Shape:
        return self.shape.replace(T=T)

    def workspace(self, shape: B.Shape) -> torch.Tensor:
        need = B.workspace_size(shape)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        return self._ws

    def new_trace(self, shape: B.Shape) -> Dict[str, torch.Tensor]:
        T, K, E, D = shape.T, shape.K, shape.E, shape.D
        od = shape.torch_dtype
        tr = {
            "logits": torch.empty(T, E, dtype=torch.float32, device="cuda"),
            "topk_ids": torch.empty(T, K, dtype=torch.int32, device="cuda"),
            "topk_w": torch.empty(T, K, dtype=torch.float32, device="cuda"),
            "counts": torch.empty(E, dtype=torch.int32, device="cuda"),
            "offsets": torch.empty(E + 1, dtype=torch.int32, device="cuda"),
            "perm_token": torch.empty(T * K, dtype=torch.int32, device="cuda"),
            "inv_pos": torch.empty(T, K, dtype=torch.int32, device="cuda"),
            "y": torch.empty(T * K, D, dtype=od, device="cuda"),
        }
        if shape.Is > 0:
            tr["shared_out"] = torch.empty(T, D, dtype=od, device="cuda")
        return tr

    def forward(self, x: torch.Tensor, mask: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                trace: bool = False, out: Optional[torch.Tensor] = None, replay_ids: Optional[torch.Tensor] = None):
        """The layer (moe_forward), or with ``replay_ids`` [T, K] int32 the
        routing replay (moe_forward_replay)."""
        shape = self.with_tokens(x.shape[0])
        od = out_dtype or torch.bfloat16
        if out is None:
            out = torch.empty(shape.T, shape.D, dtype=od, device="cuda")
        tr = self.new_trace(shape) if trace else None
        B.moe_forward(shape, self.weights, x, self.sel_bias, mask, out, self.workspace(shape), tr,
                      replay_ids=replay_ids)
        return (out, tr) if trace else out

    def forward_stages(self, x: torch.Tensor, mask: Optional[torch.Tensor] = None,
                       out_dtype: Optional[torch.dtype] = None):
        """The same layer through the four stage entry points; returns (out, boundary tensors)."""
        shape = self.with_tokens(x.shape[0])
        ws = self.workspace(shape)
        tr = self.new_trace(shape)
        B.moe_route(shape, x, self.weights["router"], self.sel_bias, mask, tr["logits"], tr["topk_ids"],
                    tr["topk_w"], ws)
        B.moe_permute(shape, tr["topk_ids"], tr["counts"], tr["offsets"], tr["perm_token"], tr["inv_pos"], ws)
        B.moe_experts(shape, x, tr["perm_token"], tr["offsets"], self.weights["gate_up"], self.weights["down"],
                      tr["y"], ws)
        shared = None
        if shape.Is > 0:
            sh_shape = shape.replace(E=1, K=1, I=shape.Is, Is=0, n_group=1, topk_group=1)
            B.moe_experts(sh_shape, x, None, None, self.weights["gate_up_shared"], self.weights["down_shared"],
                          tr["shared_out"], ws)
            shared = tr["shared_out"]
        out = torch.empty(shape.T, shape.D, dtype=out_dtype or torch.bfloat16, device="cuda")
        B.moe_combine(shape, tr["y"], tr["inv_pos"], tr["topk_w"], shared, out)
        return out, tr

    def backward(self, x: torch.Tensor, dout: torch.Tensor, trace: Dict[str, torch.Tensor],
                 mask: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
        """Gradients of the forward that produced ``trace`` (moe_backward), as
        new float32 tensors."""
        shape = self.with_tokens(x.shape[0])
        dev = x.device
        f32 = torch.float32
        S = shape
        grads = {
            "dx": torch.empty(S.T, S.D, dtype=f32, device=dev),
            "d_router": torch.empty(S.E, S.D, dtype=f32, device=dev),
            "d_gate_up": torch.empty(S.E, 2 * S.I, S.D, dtype=f32, device=dev),
            "d_down": torch.empty(S.E, S.D, S.I, dtype=f32, device=dev),
        }
        if S.Is > 0:
            grads["d_gate_up_shared"] = torch.empty(2 * S.Is, S.D, dtype=f32, device=dev)
            grads["d_down_shared"] = torch.empty(S.D, S.Is, dtype=f32, device=dev)
        ws = torch.empty(B.backward_workspace_size(shape), dtype=torch.uint8, device=dev)
        B.moe_backward(shape, self.weights, x, mask, trace, dout, grads, ws)
        return grads

