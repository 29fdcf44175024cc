"""Run the CPU oracle on inputs drawn by the synth package (tests only)."""

from typing import Optional

import numpy as np

import oracle
from synth import LayerInputs


def oracle_forward(inp: LayerInputs, tokens: Optional[np.ndarray] = None,
                   mask: Optional[np.ndarray] = None, ids_override: Optional[np.ndarray] = None):
    """The oracle forward of ``inp`` restricted to ``tokens`` (all tokens if None)."""
    cfg = inp.cfg
    x = inp.x if tokens is None else inp.x[tokens]
    if mask is None and inp.mask is not None:
        mask = inp.mask if tokens is None else inp.mask[tokens]
    return oracle.forward(
        x, inp.w_router, inp.w_gate_up, inp.w_down,
        K=cfg.K, score=cfg.score, renorm=cfg.renorm, route_scale=cfg.route_scale,
        bias=inp.bias, mask=mask,
        shared_gate_up=inp.w_gate_up_s, shared_down=inp.w_down_s,
        bf16_mode=(cfg.dtype == "bf16"), ids_override=ids_override,
        n_group=cfg.n_group, topk_group=cfg.topk_group,
    )
