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


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of the bf16 grid (8 significant bits) at |v|; 2^-133 at 0."""
    _, e = np.frexp(np.asarray(v, dtype=np.float64))   # v = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(1.0, np.where(v == 0, -133, e - 8))


def bf16_output_report(gout_bits: np.ndarray, ref64: np.ndarray, kept: Optional[np.ndarray],
                       rms: float, tol: float) -> Dict[str, float]:
    """The delivered bf16 layer output against the unrounded float64 reference.

    Counts the elements whose error exceeds ``tol * rms`` and gives the worst
    error in units of ``rms``; for every element, the distance to the
    reference rounded once to bf16 (RNE_bf16(out64)) in units of the bf16
    spacing there.  Final rounding alone can move an element by half a bf16
    ulp of its magnitude, which exceeds ``tol * rms`` only for elements of
    several RMS, so a breach that comes from the rounding sits within one ulp
    of RNE_bf16(out64); the caller asserts that.
    """
    g = as_f64(gout_bits)
    r = ref64
    if kept is not None:
        g, r = g[kept], r[kept]
    err = np.abs(g - r)
    rne = oracle.round_bf16(r)
    ulp = np.maximum(bf16_ulp(rne), bf16_ulp(g))
    dist = np.abs(g - rne) / ulp
    over = err > tol * rms
    return {
        "bf16_out_max_rel_rms": float(err.max() / rms) if err.size and rms > 0 else 0.0,
        "bf16_out_over_tol_count": int(over.sum()),
        "bf16_out_over_tol_max_dist_ulp": float(dist[over].max()) if over.any() else 0.0,
        "bf16_out_over_tol_min_abs_ref_rms": float(np.abs(r[over]).min() / rms) if over.any() else 0.0,
        "bf16_out_elements": int(err.size),
        "bf16_out_share_equal_rne": float(np.mean(dist == 0)) if err.size else 1.0,
        "bf16_out_share_within_1ulp_rne": float(np.mean(dist <= 1.0)) if err.size else 1.0,
        "bf16_out_max_dist_ulp": float(dist.max()) if err.size else 0.0,
    }


def check_layer_output(shape, tr: dict, gout: np.ndarray, ref64: np.ndarray, kept: Optional[np.ndarray],
                       tol: float, report: Optional[dict] = None,
                       tokens: Optional[np.ndarray] = None) -> Dict[str, float]:
    """Parity (c) of one layer call, both sides of the final downcast.

    The combine is run again on the call's own trace with a float32 output:
    the delivered output must be exactly that value (rounded to nearest even
    when it is bf16), and that value must lie within ``tol`` of the RMS of
    the float64 reference, with no widening.  For a bf16 output the breaches
    of ``tol * RMS`` are reported with their magnitude and each must lie
    within one bf16 ulp of the reference rounded once to bf16.  With
    ``tokens``, ``ref64`` (and ``kept``) hold those tokens only, while the
    downcast is checked on every token of ``gout``.
    """
    from routing_grouped_gemm_gemv_amd import binding as B
    T, D = gout.shape
    out32 = torch.empty(T, D, dtype=torch.float32, device="cuda")
    B.moe_combine(shape, tr["y"], tr["inv_pos"], tr["topk_w"], tr.get("shared_out"), out32)
    torch.cuda.synchronize()
    o32 = to_host(out32)
    if gout.dtype == np.uint16:
        assert np.array_equal(gout, oracle.bf16_bits_of(o32)), "bf16 output is not RNE of the float32 combine"
    else:
        assert np.array_equal(gout.view(np.uint32), o32.view(np.uint32))
    if tokens is not None:
        o32, gout = o32[tokens], gout[tokens]
    pr = dict(report or {})
    pr.update(parity_report(o32, ref64, kept))
    if gout.dtype == np.uint16:
        pr.update(bf16_output_report(gout, ref64, kept, pr["rms"], tol))
    assert pr["max_rel_rms"] <= tol, pr
    if gout.dtype == np.uint16:
        assert pr["bf16_out_over_tol_max_dist_ulp"] <= 1.0, pr
    return pr


def f32_layer(layer_bf16):
    """The same layer in the fp32-operand mode: every weight widened exactly
    from its bf16 value on the device."""
    from routing_grouped_gemm_gemv_amd import MoeLayer
    s = layer_bf16.shape.replace(dtype="f32")
    W = {k: v.float() for k, v in layer_bf16.weights.items()}
    return MoeLayer(s, W["router"], W["gate_up"], W["down"], W.get("gate_up_shared"), W.get("down_shared"),
                    layer_bf16.sel_bias)
