"""Oracle of the sparse-MoE layer backward (test infrastructure only).

The RL-Kernel roadmap ("DSV4 Flash MoE Train-Inference Consistency Roadmap":
the scope list names forward + backward with a deterministic reduction order;
the issue-bucket table asks for a single-GPU full chain, forward + backward)
puts the backward in scope without giving formulas.  The reading used here:
the gradients of the forward of ``oracle.moe.forward`` with respect to its
hidden states and weights, given the gradient G of the layer output, with

  * the top-k selection treated as fixed (a discrete choice has no gradient,
    so the selection bias gets none);
  * the bf16 rounding points of the forward passed straight through (their
    derivative taken as 1), while every product uses the values the forward
    actually used: the bf16 activation A feeds dW_down and the bf16 expert
    output y feeds the weight gradient;
  * masked tokens contributing nothing and receiving zero.

With ``grad_bf16`` the gradient operands that a bf16 GEMM would consume are
rounded to bf16 where they are formed: dY (the expert-output gradients), dH
(the gradient of the gate/up projections) and dl (the logits' gradient).  The
pages fix no precision for the backward; this option mirrors an
implementation that feeds those operands to bf16 matrix products, so that a
comparison with one isolates its accumulation order.  Without it every
gradient is the exact float64 one.

Everything is float64 (numpy matmul as the only library primitive).

For a kept token t with picks j (expert e_j, pair row p_j, weight w_j):
  out_t = sum_j w_j y_{p_j} + S_t
  dY_p   = w_j G_t                       (gradient of expert output row p)
  dw_j   = <G_t, y_p>                    (gradient of the routing weight)
  per expert e, rows R_e (gathered hidden rows X_e):
    H = X_e W1_e^T;  g = H[:, :I], u = H[:, I:];  a = silu(g) u
    dA = dY_e W2_e;  dW2_e = dY_e^T A_e
    dg = dA u silu'(g);  du = dA silu(g);  dH = [dg, du]
    dX_e = dH W1_e;  dW1_e = dH^T X_e
  shared expert: the same with dY = G on every kept token;
  router: ds over the K picks through the weights (renormalised or not, times
  route_scale), dl through the score function, dx_r = dl W_r, dW_r = dl^T x;
  dx_t = sum_j dX_{p_j} + dX_shared_t + dx_r_t.
"""

from __future__ import annotations

from typing import Callable, Dict, Optional, Tuple

import numpy as np

from .moe import expert_mlp, round_bf16, router_logits, scores, silu, widen


def sigmoid(v: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def silu_grad(v: np.ndarray) -> np.ndarray:
    """d/dv silu(v) = sigmoid(v) (1 + v (1 - sigmoid(v)))."""
    sg = sigmoid(v)
    return sg * (1.0 + v * (1.0 - sg))


def weights_grad(s: np.ndarray, ids: np.ndarray, dw: np.ndarray, renorm: bool,
                 route_scale: float) -> np.ndarray:
    """ds [T, E]: the gradient of the scores through the routing weights.

    w_j = route_scale * s_j / Z with Z = sum of the K picked scores (renorm),
    or route_scale * s_j; only picked experts receive a gradient.
    """
    T, E = s.shape
    ds = np.zeros((T, E), dtype=np.float64)
    valid = ids >= 0
    sp = np.where(valid, np.take_along_axis(s, np.maximum(ids, 0), axis=1), 0.0)
    dwv = np.where(valid, dw, 0.0)
    if renorm:
        Z = sp.sum(axis=1, keepdims=True)
        Zs = np.where(Z > 0, Z, 1.0)
        g = route_scale / Zs * (dwv - (dwv * sp).sum(axis=1, keepdims=True) / Zs)
    else:
        g = route_scale * dwv
    g = np.where(valid, g, 0.0)
    rows = np.nonzero(valid.any(axis=1))[0]
    for t in rows:
        for j in range(ids.shape[1]):
            if ids[t, j] >= 0:
                ds[t, ids[t, j]] += g[t, j]
    return ds


def score_grad(logits: np.ndarray, s: np.ndarray, ds: np.ndarray, score: str) -> np.ndarray:
    """dl [T, E]: the vector-Jacobian product of the score function."""
    if score == "softmax":
        return s * (ds - (ds * s).sum(axis=1, keepdims=True))
    if score == "sigmoid":
        return ds * s * (1.0 - s)
    if score == "sqrtsoftplus":
        # d/dl sqrt(softplus(l)) = sigmoid(l) / (2 sqrt(softplus(l)))
        with np.errstate(divide="ignore", invalid="ignore"):
            d = np.where(s > 0, sigmoid(logits) / (2.0 * np.where(s > 0, s, 1.0)), 0.0)
        return ds * d
    raise ValueError(f"unknown score function {score!r}")


def expert_mlp_backward(x64: np.ndarray, w1: np.ndarray, w2: np.ndarray, dy: np.ndarray,
                        bf16_mode: bool, grad_bf16: bool = False):
    """(dx [n, D], dW1 [2I, D], dW2 [D, I]) of one SwiGLU expert over the rows x64."""
    w1_64 = widen(w1)
    w2_64 = widen(w2)
    I = w2_64.shape[1]
    h = x64 @ w1_64.T
    g, u = h[:, :I], h[:, I:]
    a = silu(g) * u
    if bf16_mode:
        a = round_bf16(a)
    dW2 = dy.T @ a
    da = dy @ w2_64
    dg = da * u * silu_grad(g)
    du = da * silu(g)
    dh = np.concatenate([dg, du], axis=1)
    if grad_bf16:
        dh = round_bf16(dh)
    return dh @ w1_64, dh.T @ x64, dW2


def _routing_weights(x64, wr64, ids, score, renorm, route_scale):
    """Logits, scores and the routing weights [T, K] of the given picks."""
    logits = router_logits(x64, wr64)
    s = scores(logits, score)
    sp = np.where(ids >= 0, np.take_along_axis(s, np.maximum(ids, 0), axis=1), 0.0)
    if renorm:
        den = sp.sum(axis=1, keepdims=True)
        w = np.divide(sp, den, out=np.zeros_like(sp), where=den > 0) * route_scale
    else:
        w = sp * route_scale
    return logits, s, w


def _expert_step(x64, G64, w, tj, w1, w2, bf16_mode, grad_bf16):
    """(dX rows, dW1, dW2) of one expert over its picks tj = (token, slot)
    pairs in token order: dY = w G per pick, then the SwiGLU backward."""
    t_rows, j_cols = tj[:, 0], tj[:, 1]
    dy = w[t_rows, j_cols][:, None] * G64[t_rows]
    if grad_bf16:
        dy = round_bf16(dy)
    return expert_mlp_backward(x64[t_rows], w1, w2, dy, bf16_mode, grad_bf16)


def backward_expert(e: int, x: np.ndarray, w_router: np.ndarray, gate_up_e: np.ndarray, down_e: np.ndarray,
                    G: np.ndarray, ids: np.ndarray, *, score: str, renorm: bool, route_scale: float,
                    mask: Optional[np.ndarray] = None, bf16_mode: bool,
                    grad_bf16: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """(d_gate_up[e], d_down[e]) alone: the same steps as ``backward`` for the
    one expert, without the other experts, the router or dx (for sampling one
    expert's weight gradients at sizes where the full backward is too slow)."""
    x64 = widen(x)
    G64 = widen(G)
    valid = np.ones(x64.shape[0], dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    ids = np.where(valid[:, None], ids, -1)
    G64 = np.where(valid[:, None], G64, 0.0)
    _, _, w = _routing_weights(x64, widen(w_router), ids, score, renorm, route_scale)
    tj = np.argwhere(ids == e)
    I = widen(down_e).shape[1]
    if tj.size == 0:
        return np.zeros((2 * I, x64.shape[1])), np.zeros((x64.shape[1], I))
    _, dw1, dw2 = _expert_step(x64, G64, w, tj, gate_up_e, down_e, bf16_mode, grad_bf16)
    return dw1, dw2


def backward(x: np.ndarray, w_router: np.ndarray,
             gate_up: Callable[[int], np.ndarray] | np.ndarray,
             down: Callable[[int], np.ndarray] | np.ndarray,
             G: np.ndarray, ids: np.ndarray, *, score: str, renorm: bool, route_scale: float,
             mask: Optional[np.ndarray] = None,
             shared_gate_up: Optional[np.ndarray] = None, shared_down: Optional[np.ndarray] = None,
             bf16_mode: bool, grad_bf16: bool = False) -> Dict[str, np.ndarray]:
    """Gradients of the layer given the output gradient G [T, D] and the picks
    ``ids`` [T, K] (ascending, -1 for masked tokens).

    Returns float64 arrays: dx [T, D], d_router [E, D], d_gate_up [E, 2I, D],
    d_down [E, D, I], d_gate_up_shared, d_down_shared (or None), and the
    intermediate dw [T, K] (weight gradients) and dlogits [T, E].
    """
    x64 = widen(x)
    wr64 = widen(w_router)
    G64 = widen(G)
    T, D = x64.shape
    E = wr64.shape[0]
    K = ids.shape[1]
    valid = np.ones(T, dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    ids = np.where(valid[:, None], ids, -1)
    G64 = np.where(valid[:, None], G64, 0.0)

    logits, s, w = _routing_weights(x64, wr64, ids, score, renorm, route_scale)

    get1 = gate_up if callable(gate_up) else (lambda e: gate_up[e])
    get2 = down if callable(down) else (lambda e: down[e])
    I = widen(get2(0)).shape[1]
    dx = np.zeros((T, D), dtype=np.float64)
    dw = np.zeros((T, K), dtype=np.float64)
    d_gate_up = np.zeros((E, 2 * I, D), dtype=np.float64)
    d_down = np.zeros((E, D, I), dtype=np.float64)
    for e in range(E):
        tj = np.argwhere(ids == e)  # (t, j) in token order
        if tj.size == 0:
            continue
        t_rows, j_cols = tj[:, 0], tj[:, 1]
        xe = x64[t_rows]
        ye = expert_mlp(xe, get1(e), get2(e), bf16_mode)  # the y the combine used
        dw[t_rows, j_cols] = np.sum(G64[t_rows] * ye, axis=1)
        dxe, d_gate_up[e], d_down[e] = _expert_step(x64, G64, w, tj, get1(e), get2(e), bf16_mode, grad_bf16)
        np.add.at(dx, t_rows, dxe)

    d_gate_up_s = d_down_s = None
    if shared_gate_up is not None:
        dys = round_bf16(G64[valid]) if grad_bf16 else G64[valid]
        dxs, d_gate_up_s, d_down_s = expert_mlp_backward(x64[valid], shared_gate_up, shared_down,
                                                          dys, bf16_mode, grad_bf16)
        dx[valid] += dxs

    ds = weights_grad(s, ids, dw, renorm, route_scale)
    dl = score_grad(logits, s, ds, score)
    dl[~valid] = 0.0
    if grad_bf16:
        dl = round_bf16(dl)
    dx += dl @ wr64
    d_router = dl.T @ x64
    dx[~valid] = 0.0
    return {"dx": dx, "d_router": d_router, "d_gate_up": d_gate_up, "d_down": d_down,
            "d_gate_up_shared": d_gate_up_s, "d_down_shared": d_down_s, "dw": dw, "dlogits": dl}
