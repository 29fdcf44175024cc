"""Helpers shared by the GPU tests: device upload/download and parity metrics."""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

import oracle
from synth import LayerInputs


def to_dev(a: Optional[np.ndarray]) -> Optional[torch.Tensor]:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda")


def to_host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def make_layer(inp: LayerInputs):
    from routing_grouped_gemm_gemv_amd import MoeLayer, Shape
    cfg = inp.cfg
    shape = Shape(T=cfg.T, D=cfg.D, E=cfg.E, K=cfg.K, I=cfg.I, Is=cfg.Is, score=cfg.score,
                  renorm=cfg.renorm, route_scale=cfg.route_scale, dtype=cfg.dtype,
                  n_group=cfg.n_group, topk_group=cfg.topk_group)
    return MoeLayer(shape, to_dev(inp.w_router), to_dev(inp.w_gate_up), to_dev(inp.w_down),
                    to_dev(inp.w_gate_up_s), to_dev(inp.w_down_s), to_dev(inp.bias))


def as_f64(a: np.ndarray) -> np.ndarray:
    return oracle.widen(a)


def parity_report(gpu_out: np.ndarray, ref64: np.ndarray, kept: Optional[np.ndarray] = None) -> Dict[str, float]:
    """max-abs error relative to the reference RMS, with drift percentiles."""
    g = as_f64(gpu_out)
    r = ref64
    if kept is not None:
        g = g[kept]
        r = r[kept]
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(g - r)
    rep = {
        "token_count": int(g.shape[0]),
        "rms": rms,
        "max_absdiff": float(err.max()) if err.size else 0.0,
        "max_rel_rms": float(err.max() / rms) if err.size and rms > 0 else 0.0,
    }
    if err.size:
        for q in (50, 99, 99.99):
            rep[f"p{q}_rel_rms"] = float(np.percentile(err, q) / rms) if rms > 0 else 0.0
    return rep


def routing_check(gpu_ids: np.ndarray, ref) -> Dict[str, object]:
    """Top-k ids: bit-exact except tokens with a near tie at the K boundary."""
    same = np.all(gpu_ids == ref.ids, axis=1)
    exempt = ref.exempt
    bad = np.nonzero(~same & ~exempt)[0]
    return {
        "token_count": int(gpu_ids.shape[0]),
        "exempt_count": int(exempt.sum()),
        "exempt_tokens": np.nonzero(exempt)[0].tolist()[:50],
        "exempt_differing": int((~same & exempt).sum()),
        "mismatch_count": int(bad.size),
        "mismatch_tokens": bad.tolist()[:20],
    }
