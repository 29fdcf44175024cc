"""Oracle of the sparse-MoE layer forward (test infrastructure only).

Sources, cited by page title and section:
  [RLK]  RL-Kernel blog, "DSV4 Flash MoE Train-Inference Consistency Roadmap":
         "Problem 1: Routing Is A Discrete Decision", "Problem 2: Single-Operator
         Boundaries May Not Be Meaningful" (the semantic boundaries: routing,
         dispatch, expert, shared-expert, reduction), "Problem 3: Final Reduction
         Is The Core Drift Point", "R3 Should Not Be A Prerequisite".
  [ARX]  arXiv 2607.28097, "From Expert Reduction to Behavioral Divergence:
         Tracing Numerical State through Sparse MoE Inference", Abstract.
  [SPF]  SpecForge pull request #1003, "MoE FFN support for DFlash-family drafts":
         "Design notes", "Out of scope", "Revised version" and the commit notes
         on the router (selection bias, top-k weights, token mask).

Conventions (the plainest reading where the pages leave a step open):
  * logits are x . W_r^T; scores are softmax over the experts or the logistic
    sigmoid of each logit;
  * the selection bias is added to the scores to rank experts ("choice"), and
    the weights are taken from the unbiased scores [SPF, router commit notes];
  * the K experts with the largest choice are selected, ties going to the lower
    expert id; the K ids of a token are returned in ascending id order;
  * the pages name two more score functions and a select override without
    formulas [SPF, commit notes on the load-balance loss and on select]:
    sqrtsoftplus is read as sqrt(softplus(l)) = sqrt(log(1 + e^l)), and the
    DeepSeek-V3 group-limited select as: the E experts form n_group groups of
    E/n_group consecutive ids, a group's score is the sum of its two largest
    choices, the topk_group best groups (ties to the lower group id) are
    kept, and the K experts are chosen from the kept groups only;
  * weights are renormalised over the selected experts when ``renorm`` is set,
    then multiplied by ``route_scale`` [SPF, "Revised version", "Out of scope"];
  * masked tokens take no route, no expert work and produce a zero row;
  * an expert is a SwiGLU MLP: gate and up projections (rows 0..I-1 and
    I..2I-1 of the [2I, D] gate_up matrix), silu(gate) * up, then the [D, I]
    down projection [RLK, Problem 2: gate_and_up -> down];
  * in the bf16 operand mode the activation fed to the down projection is a
    bf16 operand (rounded nearest-even, one rounding from the exact value) and
    the expert output crosses the expert boundary as bf16; in the fp32 mode
    nothing is rounded;
  * the reference layer output is the float64 sum of the weighted exact expert
    outputs (before their bf16 conversion) and the exact shared output: the
    conversion itself belongs to the combine, whose arithmetic is emulated
    bit for bit separately;
  * the shared expert is the same MLP applied to every kept token, ungated,
    added after the routed terms [SPF, "Design notes"];
  * the combine accumulates in float32, from +0, over the K routed terms in
    ascending expert id, each term the float32 product of the float32 weight
    and the widened expert output, then adds the shared output, then rounds to
    bf16 [RLK, Problem 3; ARX, Abstract];
  * the order-invariant combine mode forms the same products exactly in
    float64, sums them and the shared output in float64 in the same order and
    rounds once (a reduction whose result does not depend on the order of the
    terms whenever that sum is exact, the property [ARX, Abstract] measures
    order dependence against).
"""

from __future__ import annotations

import itertools
from dataclasses import dataclass, field
from typing import Callable, Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

# The exemption threshold on the oracle's relative margin between the K-th and
# (K+1)-th choice: tokens strictly between 0 and this margin may legitimately
# pick a different K-th expert in another correct implementation.
EXEMPT_REL_MARGIN = 1e-6


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------

def widen(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or float32 values -> float64, exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported operand dtype {a.dtype}")


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the bf16 grid (8 significant bits), nearest-even.

    One rounding from the float64 value (not float64 -> float32 -> bf16).  The
    values here are far inside bf16's normal range, so no overflow or subnormal
    handling is needed.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                 # v = m * 2^e with 0.5 <= |m| < 1
    q = np.ldexp(m, 8)                 # 128 <= |q| < 256: the integer significand grid
    return np.ldexp(np.rint(q), e - 8)  # rint rounds halves to even


def bf16_bits_of(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values (float32 or float64) rounded nearest-even."""
    r = round_bf16(np.asarray(v, dtype=np.float64)).astype(np.float32)  # exact: on the bf16 grid
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _f32_of(a: np.ndarray) -> np.ndarray:
    """bf16 bits or float32 values -> float32, exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if a.dtype == np.float32:
        return a
    raise TypeError(f"unsupported expert-output dtype {a.dtype}")


# ----------------------------------------------------------------------------
# routing boundary: logits, scores, choice, top-k ids, top-k weights
# [RLK, Problem 1 and the routing boundary of Problem 2]
# ----------------------------------------------------------------------------

def router_logits(x64: np.ndarray, wr64: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_d x[t, d] * W_r[e, d], float64."""
    return x64 @ wr64.T


def silu(v: np.ndarray) -> np.ndarray:
    """silu(v) = v * logistic(v) = v / (1 + exp(-v)), float64."""
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def scores(logits: np.ndarray, score: str) -> np.ndarray:
    """Router scores in float64: softmax over experts, the logistic sigmoid, or
    sqrtsoftplus, sqrt(log(1 + e^l)) of each logit [SPF, commit notes]."""
    if score == "softmax":
        z = logits - logits.max(axis=1, keepdims=True)
        ez = np.exp(z)
        return ez / ez.sum(axis=1, keepdims=True)
    if score == "sigmoid":
        with np.errstate(over="ignore"):
            return 1.0 / (1.0 + np.exp(-logits))
    if score == "sqrtsoftplus":
        # log(1 + e^l) = max(l, 0) + log(1 + e^-|l|): the same value, no overflow
        return np.sqrt(np.maximum(logits, 0.0) + np.log1p(np.exp(-np.abs(logits))))
    raise ValueError(f"unknown score function {score!r}")


def select_topk(choice: np.ndarray, K: int, valid: Optional[np.ndarray] = None
                ) -> Tuple[np.ndarray, np.ndarray]:
    """Top-K experts per token under the order (choice descending, id ascending).

    Returns (ids [T, K] int32 in ascending id order, -1 for masked tokens;
    rel_margin [T] float64 = (c_K - c_{K+1}) / max(|c_K|, |c_{K+1}|) of the
    sorted choices, +inf when K == E or the token is masked).
    """
    T, E = choice.shape
    # a stable ascending sort of -choice keeps equal choices in id order
    order = np.argsort(-choice, axis=1, kind="stable")
    ids = np.sort(order[:, :K], axis=1).astype(np.int32)
    margin = np.full(T, np.inf)
    if K < E:
        ck = np.take_along_axis(choice, order[:, K - 1:K], axis=1)[:, 0]
        ck1 = np.take_along_axis(choice, order[:, K:K + 1], axis=1)[:, 0]
        margin = _rel_margin(ck, ck1)
    if valid is not None:
        ids[~valid] = -1
        margin[~valid] = np.inf
    return ids, margin


def _rel_margin(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """(a - b) / max(|a|, |b|) for a >= b; +inf where b is -inf (nothing else
    competes), 0 where both are 0."""
    den = np.maximum(np.abs(a), np.abs(b))
    with np.errstate(invalid="ignore", divide="ignore"):
        m = np.where(den > 0, (a - b) / np.where(den > 0, den, 1.0), 0.0)
    return np.where(np.isneginf(b), np.inf, m)


def select_grouped(choice: np.ndarray, K: int, n_group: int, topk_group: int,
                   valid: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Group-limited top-K, the DeepSeek-V3 select the pages name [SPF, commit
    notes on select], read as: group g holds experts g*E/n_group ..
    (g+1)*E/n_group - 1; its score is the sum of its two largest choices; the
    topk_group groups with the largest scores are kept (ties to the lower
    group id); the K experts are then chosen among the kept groups' experts
    as select_topk chooses them.

    Returns (ids, rel_margin) like select_topk; rel_margin is the smaller of
    the expert margin among the kept experts and the group margin between the
    topk_group-th and the next group score, since a near tie in either
    decision may flip a pick.
    """
    T, E = choice.shape
    gs = E // n_group
    cg = choice.reshape(T, n_group, gs)
    top2 = -np.sort(-cg, axis=2)[:, :, :2]
    gscore = top2[:, :, 0] + top2[:, :, 1]
    gorder = np.argsort(-gscore, axis=1, kind="stable")
    kept = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(kept, gorder[:, :topk_group], True, axis=1)
    allowed = np.repeat(kept, gs, axis=1)
    ids, margin = select_topk(np.where(allowed, choice, -np.inf), K, valid)
    if topk_group < n_group:
        gk = np.take_along_axis(gscore, gorder[:, topk_group - 1:topk_group], axis=1)[:, 0]
        gk1 = np.take_along_axis(gscore, gorder[:, topk_group:topk_group + 1], axis=1)[:, 0]
        gm = _rel_margin(gk, gk1)
        if valid is not None:
            gm = np.where(valid, gm, np.inf)
        margin = np.minimum(margin, gm)
    return ids, margin


def topk_weights(s: np.ndarray, ids: np.ndarray, renorm: bool, route_scale: float) -> np.ndarray:
    """Weights from the unbiased scores of the selected experts, float64.

    w_j = s[t, id_j]; if renorm, w_j /= sum of the selected scores; then
    w_j *= route_scale.  Masked tokens (ids -1) get weight 0.
    """
    valid = ids >= 0
    w = np.where(valid, np.take_along_axis(s, np.maximum(ids, 0), axis=1), 0.0)
    if renorm:
        den = w.sum(axis=1, keepdims=True)
        w = np.divide(w, den, out=np.zeros_like(w), where=den > 0)
    return w * route_scale


# ----------------------------------------------------------------------------
# dispatch boundary: per-expert counts, offsets, stable permutation
# [RLK, Problem 2: token-to-expert map, valid token counts, padding provenance]
# ----------------------------------------------------------------------------

def permute(ids: np.ndarray, E: int) -> Dict[str, np.ndarray]:
    """Counting sort of the (token, slot) pairs by expert, stable in token order.

    counts[e]      number of kept pairs routed to e
    offsets[e]     exclusive prefix sum of counts (offsets[E] = kept pairs)
    perm_token[p]  the token of the p-th row of the expert-sorted order
    inv_pos[t, j]  the row of pair (t, j) in that order (-1 for masked)
    """
    T, K = ids.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(K):
            if ids[t, j] >= 0:
                counts[ids[t, j]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    nxt = offsets[:E].copy()
    perm_token = np.empty(int(offsets[E]), dtype=np.int64)
    inv_pos = np.full((T, K), -1, dtype=np.int64)
    for t in range(T):
        for j in range(K):
            e = ids[t, j]
            if e < 0:
                continue
            p = nxt[e]
            nxt[e] += 1
            perm_token[p] = t
            inv_pos[t, j] = p
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "perm_token": perm_token.astype(np.int32),
        "inv_pos": inv_pos.astype(np.int32),
    }


# ----------------------------------------------------------------------------
# expert boundary [RLK, Problem 2: expert inputs/outputs, accumulation dtype]
# ----------------------------------------------------------------------------

def expert_mlp(x64: np.ndarray, w1: np.ndarray, w2: np.ndarray, bf16_mode: bool,
               exact_output: bool = False) -> np.ndarray:
    """One SwiGLU expert on the rows of x64, float64.

    h = x . W1^T ([n, 2I]); a = silu(h[:, :I]) * h[:, I:]; y = a . W2^T ([n, D]).
    In bf16 mode a is rounded to bf16 (nearest-even) before the down projection
    and y is returned on the bf16 grid, unless ``exact_output`` asks for the
    value before that last conversion.
    """
    w1_64 = widen(w1)
    w2_64 = widen(w2)
    I = w2_64.shape[1]
    assert w1_64.shape[0] == 2 * I
    h = x64 @ w1_64.T
    a = silu(h[:, :I]) * h[:, I:]
    if bf16_mode:
        a = round_bf16(a)
    y = a @ w2_64.T
    if bf16_mode and not exact_output:
        y = round_bf16(y)
    return y


# ----------------------------------------------------------------------------
# reduction boundary: the weighted combine
# [RLK, Problem 3; ARX, Abstract: operand conversion, accumulator precision and
#  reduction order are part of the numerical contract]
# ----------------------------------------------------------------------------

def combine_fp32(y: np.ndarray, inv_pos: np.ndarray, w32: np.ndarray,
                 shared: Optional[np.ndarray] = None, order: Optional[Sequence[int]] = None,
                 out: str = "bf16") -> np.ndarray:
    """Float32 emulation of the combine, one IEEE rounding per operation.

    acc = +0; for j in ``order`` (default 0..K-1, i.e. ascending expert id):
    p = fl32(w[t, j] * f32(y[inv_pos[t, j]])); acc = fl32(acc + p).  Then
    acc = fl32(acc + f32(shared[t])) if a shared output is given.  Masked tokens
    (inv_pos -1) give a +0 row.  ``out`` = "bf16" returns bf16 bit patterns
    (nearest-even), "f32" returns the float32 accumulator.
    """
    T, K = inv_pos.shape
    y32 = _f32_of(y)
    D = y32.shape[1] if y32.ndim == 2 else (_f32_of(shared).shape[1])
    w32 = np.asarray(w32, dtype=np.float32)
    order = range(K) if order is None else order
    kept = (inv_pos >= 0).any(axis=1) if K > 0 else np.zeros(T, dtype=bool)
    acc = np.zeros((T, D), dtype=np.float32)
    for j in order:
        rows = inv_pos[:, j]
        yj = np.zeros((T, D), dtype=np.float32)
        yj[rows >= 0] = y32[rows[rows >= 0]]
        p = w32[:, j:j + 1] * yj        # float32 x float32 -> float32, rounded
        acc = acc + p                   # float32 + float32 -> float32, rounded
    if shared is not None:
        acc = acc + _f32_of(shared)
    acc[~kept] = 0.0
    if out == "f32":
        return acc
    return bf16_bits_of(acc)


def combine_f64(y: np.ndarray, inv_pos: np.ndarray, w32: np.ndarray,
                shared: Optional[np.ndarray] = None, order: Optional[Sequence[int]] = None,
                out: str = "bf16") -> np.ndarray:
    """The order-invariant combine: the terms in float64, rounded once.

    Each product w[t, j] * y[inv_pos[t, j]] of a float32 weight and a bf16 (or
    float32) expert output is exact in float64; acc = +0; for j in ``order``
    (default ascending expert id): acc = fl64(acc + product); then acc =
    fl64(acc + shared[t]); the result is acc rounded once, nearest-even, to
    bf16 (``out`` = "bf16", bit patterns) or float32 (``out`` = "f32").  When
    the float64 sum is exact the order of the terms does not matter: the
    order-invariant reduction the reduction-order results of [ARX, Abstract]
    motivate.  Masked tokens (inv_pos -1) give a +0 row.
    """
    T, K = inv_pos.shape
    y64 = widen(y)
    D = y64.shape[1] if y64.ndim == 2 else widen(shared).shape[1]
    w64 = np.asarray(w32, dtype=np.float32).astype(np.float64)
    order = range(K) if order is None else order
    kept = (inv_pos >= 0).any(axis=1) if K > 0 else np.zeros(T, dtype=bool)
    acc = np.zeros((T, D), dtype=np.float64)
    for j in order:
        rows = inv_pos[:, j]
        yj = np.zeros((T, D), dtype=np.float64)
        yj[rows >= 0] = y64[rows[rows >= 0]]
        acc = acc + w64[:, j:j + 1] * yj   # the product is exact; one rounding per add
    if shared is not None:
        acc = acc + widen(shared)
    acc[~kept] = 0.0
    if out == "f32":
        return acc.astype(np.float32)      # one rounding, nearest-even
    return bf16_bits_of(acc)               # one rounding from float64


def combine_orders(y: np.ndarray, inv_pos: np.ndarray, w32: np.ndarray,
                   shared: Optional[np.ndarray] = None,
                   orders: Optional[Iterable[Sequence[int]]] = None,
                   mode: str = "f32") -> Dict[Tuple[int, ...], np.ndarray]:
    """The combine (float32 output) for each order of the K routed terms.

    Default: all K! permutations (720 for the six routed terms of [ARX]).
    ``mode`` "f32" is the float32 fold, "f64" the order-invariant sum.
    """
    K = inv_pos.shape[1]
    orders = itertools.permutations(range(K)) if orders is None else orders
    fn = combine_f64 if mode == "f64" else combine_fp32
    return {tuple(o): fn(y, inv_pos, w32, shared, order=o, out="f32") for o in orders}


# ----------------------------------------------------------------------------
# the whole layer
# ----------------------------------------------------------------------------

@dataclass
class RouteResult:
    logits: np.ndarray        # [T, E] float64
    scores: np.ndarray        # [T, E] float64
    choice: np.ndarray        # [T, E] float64
    ids: np.ndarray           # [T, K] int32, ascending, -1 masked
    weights: np.ndarray       # [T, K] float64
    rel_margin: np.ndarray    # [T] float64
    exempt: np.ndarray        # [T] bool: 0 < rel_margin < EXEMPT_REL_MARGIN


def route(x: np.ndarray, w_router: np.ndarray, *, K: int, score: str, renorm: bool, route_scale: float,
          bias: Optional[np.ndarray] = None, mask: Optional[np.ndarray] = None,
          ids_override: Optional[np.ndarray] = None, n_group: int = 1, topk_group: int = 1) -> RouteResult:
    """The routing boundary alone [RLK, Problem 1]: logits, scores, choice,
    top-K ids (ascending, -1 for masked tokens), weights and the near-tie
    margin, exactly as ``forward`` computes them.  ``ids_override`` replays
    given ids [RLK, "R3 Should Not Be A Prerequisite"]; the weights then come
    from the scores of those ids."""
    x64 = widen(x)
    wr64 = widen(w_router)
    T = x64.shape[0]
    valid = np.ones(T, dtype=bool) if mask is None else np.asarray(mask).astype(bool)

    logits = router_logits(x64, wr64)
    s = scores(logits, score)
    c = s + widen(bias)[None, :] if bias is not None else s
    if n_group > 1:
        ids, margin = select_grouped(c, K, n_group, topk_group, valid)
    else:
        ids, margin = select_topk(c, K, valid)
    if ids_override is not None:
        ids = np.asarray(ids_override, dtype=np.int32).copy()
        ids[~valid] = -1
    w = topk_weights(s, ids, renorm, route_scale)
    exempt = (margin > 0) & (margin < EXEMPT_REL_MARGIN)
    return RouteResult(logits, s, c, ids, w, margin, exempt)


@dataclass
class OracleResult:
    logits: np.ndarray        # [T, E] float64
    scores: np.ndarray        # [T, E] float64
    choice: np.ndarray        # [T, E] float64
    ids: np.ndarray           # [T, K] int32, ascending, -1 masked
    weights: np.ndarray       # [T, K] float64
    rel_margin: np.ndarray    # [T] float64
    exempt: np.ndarray        # [T] bool: 0 < rel_margin < EXEMPT_REL_MARGIN
    counts: np.ndarray        # [E] int32
    offsets: np.ndarray       # [E+1] int32
    perm_token: np.ndarray    # [P] int32
    inv_pos: np.ndarray       # [T, K] int32
    y: np.ndarray             # [P, D] float64 expert outputs at the boundary (bf16 grid in bf16 mode)
    shared: Optional[np.ndarray]  # [T, D] float64 shared output at the boundary, or None
    out: np.ndarray           # [T, D] float64 reference: sum_j w_j y_exact_j + shared_exact
    y_exact: Optional[np.ndarray] = None       # [P, D] expert outputs before the bf16 conversion
    shared_exact: Optional[np.ndarray] = None  # [T, D]
    extra: Dict[str, object] = field(default_factory=dict)


def forward(x: np.ndarray, w_router: np.ndarray,
            gate_up: Callable[[int], np.ndarray] | np.ndarray,
            down: Callable[[int], np.ndarray] | np.ndarray,
            *, K: int, score: str, renorm: bool, route_scale: float,
            bias: Optional[np.ndarray] = None, mask: Optional[np.ndarray] = None,
            shared_gate_up: Optional[np.ndarray] = None, shared_down: Optional[np.ndarray] = None,
            bf16_mode: bool, ids_override: Optional[np.ndarray] = None,
            n_group: int = 1, topk_group: int = 1) -> OracleResult:
    """The layer forward on the CPU, every boundary tensor returned.

    ``gate_up``/``down`` are the stacked expert weights ([E, 2I, D], [E, D, I])
    or callables returning expert e's matrices.  ``ids_override`` replays given
    top-k ids (ascending, -1 masked) instead of selecting them, as the routing
    replay of [RLK, "R3 Should Not Be A Prerequisite"] does; the weights then
    come from the oracle's own scores of those ids.  ``n_group`` > 1 selects
    with select_grouped.
    """
    x64 = widen(x)
    T = x64.shape[0]
    E = np.asarray(w_router).shape[0]
    valid = np.ones(T, dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    rt = route(x64, w_router, K=K, score=score, renorm=renorm, route_scale=route_scale, bias=bias, mask=mask,
               ids_override=ids_override, n_group=n_group, topk_group=topk_group)
    logits, s, c, ids, w, margin, exempt = (rt.logits, rt.scores, rt.choice, rt.ids, rt.weights,
                                            rt.rel_margin, rt.exempt)

    pm = permute(ids, E)
    offsets = pm["offsets"]
    perm_token = pm["perm_token"]
    D = x64.shape[1]
    y_ex = np.zeros((int(offsets[E]), D), dtype=np.float64)
    get1 = gate_up if callable(gate_up) else (lambda e: gate_up[e])
    get2 = down if callable(down) else (lambda e: down[e])
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y_ex[lo:hi] = expert_mlp(x64[perm_token[lo:hi]], get1(e), get2(e), bf16_mode, exact_output=True)
    y = round_bf16(y_ex) if bf16_mode else y_ex

    sh = sh_ex = None
    if shared_gate_up is not None:
        sh_ex = np.zeros((T, D), dtype=np.float64)
        if valid.any():
            sh_ex[valid] = expert_mlp(x64[valid], shared_gate_up, shared_down, bf16_mode, exact_output=True)
        sh = round_bf16(sh_ex) if bf16_mode else sh_ex

    out = np.zeros((T, D), dtype=np.float64)
    inv_pos = pm["inv_pos"]
    for j in range(K):
        rows = inv_pos[:, j]
        ok = rows >= 0
        out[ok] += w[ok, j:j + 1] * y_ex[rows[ok]]
    if sh_ex is not None:
        out += sh_ex
    out[~valid] = 0.0
    return OracleResult(logits, s, c, ids, w, margin, exempt, pm["counts"], offsets,
                        perm_token, inv_pos, y, sh, out, y_ex, sh_ex)
