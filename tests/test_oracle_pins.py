"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one oracle function to an independent statement of the same
fact: exact rational arithmetic, a library routine, a brute-force search, a
closed form, or a number the pages print.
"""

import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs
from synth.configs import TIE_TOKENS
from tests.oracle_bridge import oracle_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- exact rounding

def _round_rational(q: Fraction, p: int) -> Fraction:
    """Round a rational to p significant bits, ties to even (normal range only)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length() - p
    while a / Fraction(2) ** e >= 2 ** p:
        e += 1
    while a / Fraction(2) ** e < 2 ** (p - 1):
        e -= 1
    m = a / Fraction(2) ** e
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * Fraction(2) ** e


def _r32(q):
    return _round_rational(q, 24)


def _rbf16(q):
    return _round_rational(q, 8)


def test_round_bf16_matches_exact_rational():
    rng = np.random.default_rng(11)
    vals = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000))
    # exact midpoints between neighbouring bf16 values, with even and odd lower neighbour
    for sig in (128, 129, 200, 201, 254, 255):
        for ex in (-20, -3, 0, 5):
            vals.append((sig + 0.5) * 2.0 ** ex)
            vals.append(-(sig + 0.5) * 2.0 ** ex)
    v = np.array(vals, dtype=np.float64)
    got = oracle.round_bf16(v)
    for a, g in zip(v, got):
        assert Fraction(float(g)) == _rbf16(Fraction(float(a)))


def test_round_bf16_is_one_rounding_from_float64():
    # (129 + 1/2 + 2^-30) * 2^-7 lies just above a bf16 midpoint: a direct rounding goes
    # up to 130, while rounding to float32 first lands exactly on the midpoint and then
    # rounds to the even neighbour 129.
    v = np.array([(129.5 + 2.0 ** -30) * 2.0 ** -7])
    assert float(np.float32(v[0])) == 129.5 * 2.0 ** -7
    assert oracle.round_bf16(v)[0] == 130.0 * 2.0 ** -7


def test_bf16_bits_match_torch_cast():
    rng = np.random.default_rng(12)
    a = (rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000)).astype(np.float32)
    bits = a.view(np.uint32)
    # force many exact float32 -> bf16 ties
    a2 = ((bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    for arr in (a, a2):
        ours = oracle.bf16_bits_of(arr)
        ref = torch.from_numpy(arr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(ours, ref)


# ---------------------------------------------------------------- routing

def test_router_logits_match_exact_rational():
    cfg = get_config("tiny")
    inp = make_inputs(cfg)
    x64, wr64 = oracle.widen(inp.x), oracle.widen(inp.w_router)
    lg = oracle.router_logits(x64, wr64)
    D = cfg.D
    u = 2.0 ** -53
    gamma = D * u / (1 - D * u)
    for t in (0, 1, 2, 40, 63):
        for e in range(cfg.E):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x64[t], wr64[e]))
            bound = gamma * float(np.sum(np.abs(x64[t] * wr64[e])))
            assert abs(Fraction(float(lg[t, e])) - exact) <= Fraction(bound)
    # one-hot and zero rows: logits are exactly a router column, or exactly zero
    assert np.all(lg[5] == 0.0)
    for t, col in ((17, 0), (33, 1), (60, 2)):
        np.testing.assert_array_equal(lg[t], wr64[:, col])


def test_scores_match_torch():
    rng = np.random.default_rng(13)
    lg = rng.standard_normal((64, 256)) * 3.0
    sm = oracle.scores(lg, "softmax")
    sg = oracle.scores(lg, "sigmoid")
    np.testing.assert_allclose(sm, torch.softmax(torch.from_numpy(lg), dim=1).numpy(), rtol=1e-13, atol=0)
    np.testing.assert_allclose(sg, torch.sigmoid(torch.from_numpy(lg)).numpy(), rtol=1e-13, atol=0)
    with pytest.raises(ValueError):
        oracle.scores(lg, "relu")


def test_sqrtsoftplus_matches_torch_and_closed_forms():
    # torch's softplus (library routine; a threshold beyond reach keeps its
    # log1p(exp(l)) formula, which overflows past l ~ 709), then sqrt
    lg = np.concatenate([np.linspace(-700, 700, 2801), np.random.default_rng(15).standard_normal(2000) * 4])[None, :]
    ss = oracle.scores(lg, "sqrtsoftplus")
    ref = torch.nn.functional.softplus(torch.from_numpy(lg), beta=1.0, threshold=1e300).sqrt().numpy()
    np.testing.assert_allclose(ss, ref, rtol=1e-14, atol=1e-300)
    # closed forms: sqrt(log 2) at 0; sqrt(l) up to e^-l / (2 sqrt(l)) for large l; sqrt(e^l) for very negative l
    z = oracle.scores(np.array([[0.0, 60.0, -60.0, 1000.0]]), "sqrtsoftplus")[0]
    assert abs(z[0] - np.sqrt(np.log(2.0))) <= 1e-16
    assert abs(z[1] - np.sqrt(60.0)) <= 1e-15 * np.sqrt(60.0)
    assert abs(z[2] - np.exp(-30.0)) <= 1e-14 * np.exp(-30.0)
    assert z[3] == np.sqrt(1000.0)
    assert np.all(np.diff(oracle.scores(np.linspace(-20, 20, 401)[None, :], "sqrtsoftplus")[0]) > 0)


def _golden_grouped():
    with open(os.path.join(GOLDEN, "grouped_select_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", range(3))
def test_select_grouped_hand_examples(case):
    c = _golden_grouped()[case]
    choice = np.array([c["choice"]], dtype=np.float64)
    ids, _ = oracle.select_grouped(choice, c["K"], c["n_group"], c["topk_group"])
    assert list(ids[0]) == c["ids"]
    ids0, _ = oracle.select_topk(choice, c["K"])
    assert list(ids0[0]) == c["ungrouped_ids"]


def _grouped_brute(row, K, G, TG):
    """Plain Python lists: group scores, kept groups, then the dominance rule."""
    E = len(row)
    gs = E // G
    gscore = []
    for g in range(G):
        vals = sorted(row[g * gs:(g + 1) * gs], reverse=True)
        gscore.append(vals[0] + vals[1])
    kept = sorted(range(G), key=lambda g: (-gscore[g], g))[:TG]
    allowed = [e for e in range(E) if e // gs in kept]
    picks = sorted(allowed, key=lambda e: (-row[e], e))[:K]
    return sorted(picks), kept


@pytest.mark.parametrize("E,G,TG,K", [(8, 4, 2, 3), (16, 4, 1, 2), (32, 8, 4, 6), (24, 3, 2, 5)])
def test_select_grouped_matches_brute_force(E, G, TG, K):
    rng = np.random.default_rng(E * 100 + G * 10 + TG)
    c = rng.integers(-3, 4, size=(400, E)) / 4.0   # many exact ties, in groups and across them
    ids, _ = oracle.select_grouped(c, K, G, TG)
    for t in range(c.shape[0]):
        picks, kept = _grouped_brute(list(c[t]), K, G, TG)
        assert list(ids[t]) == picks
        assert all(e // (E // G) in kept for e in ids[t])


def test_select_grouped_reductions():
    rng = np.random.default_rng(21)
    c = rng.standard_normal((300, 64))
    base, m0 = oracle.select_topk(c, 6)
    for G, TG in ((1, 1), (8, 8), (4, 4)):
        ids, m = oracle.select_grouped(c, 6, G, TG)
        np.testing.assert_array_equal(ids, base)
        np.testing.assert_array_equal(m, m0)
    # one group kept: all picks inside the best group
    ids, _ = oracle.select_grouped(c, 2, 8, 1)
    assert np.all(ids[:, 0] // 8 == ids[:, 1] // 8)


def test_select_grouped_margin_covers_group_ties():
    # groups 1 and 3 tie exactly (0.9375): not exempt (an exact tie); raise
    # group 3 by 2^-50 (the sum keeps it): exempt, and group 3 now wins
    c = np.array([_golden_grouped()[0]["choice"]], dtype=np.float64)
    _, m = oracle.select_grouped(c, 3, 4, 2)
    assert m[0] == 0.0
    c2 = c.copy()
    c2[0, 6] = 0.25 + 2.0 ** -50
    ids, m2 = oracle.select_grouped(c2, 3, 4, 2)
    assert 0 < m2[0] < oracle.EXEMPT_REL_MARGIN
    assert list(ids[0]) == [0, 6, 7]


def test_silu_matches_torch():
    v = np.concatenate([np.linspace(-800, 800, 4001), np.random.default_rng(14).standard_normal(1000)])
    np.testing.assert_allclose(oracle.silu(v), torch.nn.functional.silu(torch.from_numpy(v)).numpy(),
                               rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("K", [1, 2, 3, 5, 8])
def test_select_topk_matches_dominance_count(K):
    E = 8
    rng = np.random.default_rng(100 + K)
    c = rng.integers(0, 4, size=(500, E)) / 4.0   # many exact ties
    ids, _ = oracle.select_topk(c, K)
    for t in range(c.shape[0]):
        rank = [sum(1 for j in range(E) if c[t, j] > c[t, e] or (c[t, j] == c[t, e] and j < e))
                for e in range(E)]
        brute = sorted(e for e in range(E) if rank[e] < K)
        assert list(ids[t]) == brute


def test_select_topk_matches_exhaustive_subsets():
    E, K = 8, 3
    rng = np.random.default_rng(7)
    c = rng.integers(-2, 3, size=(200, E)).astype(np.float64)
    ids, _ = oracle.select_topk(c, K)

    def beats(t, i, j):
        return c[t, i] > c[t, j] or (c[t, i] == c[t, j] and i < j)

    for t in range(c.shape[0]):
        good = [S for S in itertools.combinations(range(E), K)
                if all(beats(t, i, j) for i in S for j in range(E) if j not in S)]
        assert len(good) == 1
        assert tuple(ids[t]) == good[0]


def test_negative_zero_ties_positive_zero():
    c = np.array([[0.0, -0.0, -0.0, 0.0, -1.0]])
    ids, margin = oracle.select_topk(c, 2)
    assert list(ids[0]) == [0, 1]
    assert margin[0] == 0.0


def test_tiny_tie_tokens_closed_form():
    cfg = get_config("tiny")
    res = oracle_forward(make_inputs(cfg))
    # token 5: zero row, eight-way tie -> the two lowest ids, weights exactly 1/2
    assert list(res.ids[5]) == [0, 1]
    assert list(res.weights[5]) == [0.5, 0.5]
    # token 17: expert 1 first, experts 2 and 3 tie for rank 2 -> {1, 2}
    assert list(res.ids[17]) == [1, 2]
    # token 33: experts 1 and 3 tie at the top -> {1, 3}, equal weights
    assert list(res.ids[33]) == [1, 3]
    assert res.weights[33, 0] == res.weights[33, 1] == 0.5
    # token 60: expert 0 first, experts 2, 4, 6 tie for rank 2 -> {0, 2}
    assert list(res.ids[60]) == [0, 2]
    # ties across the K-th/(K+1)-th boundary have zero margin and are never exempt;
    # token 33's tie sits inside the top-2, so its boundary margin is positive
    for t in (5, 17, 60):
        assert res.rel_margin[t] == 0.0
    assert res.rel_margin[33] > 1e-3
    assert not res.exempt[list(TIE_TOKENS)].any()


def test_exemption_flags_near_ties_only():
    c = np.array([[1.0, 1.0 - 5e-7, 0.5],       # rel margin 5e-7: exempt
                  [1.0, 1.0 - 5e-6, 0.5],       # 5e-6: not exempt
                  [1.0, 1.0, 0.5]])             # exact tie: not exempt
    _, m = oracle.select_topk(c, 1)
    ex = (m > 0) & (m < oracle.EXEMPT_REL_MARGIN)
    assert list(ex) == [True, False, False]
    np.testing.assert_allclose(m[:2], [5e-7, 5e-6], rtol=1e-9)


def test_weights_sum_to_route_scale():
    rng = np.random.default_rng(15)
    s = oracle.scores(rng.standard_normal((300, 256)), "sigmoid")
    ids, _ = oracle.select_topk(s + rng.uniform(-0.05, 0.05, 256)[None, :], 6)
    w = oracle.topk_weights(s, ids, True, 2.5)
    np.testing.assert_allclose(w.sum(axis=1), 2.5, rtol=0, atol=1e-12)
    # weights come from the unbiased scores
    np.testing.assert_allclose(w / 2.5 * np.take_along_axis(s, ids, 1).sum(1, keepdims=True),
                               np.take_along_axis(s, ids, 1), rtol=1e-13)


def test_top1_renorm_is_one_and_zero_row_is_uniform():
    rng = np.random.default_rng(16)
    s = oracle.scores(rng.standard_normal((50, 16)), "softmax")
    ids, _ = oracle.select_topk(s, 1)
    assert np.all(oracle.topk_weights(s, ids, True, 1.0) == 1.0)
    for K in (1, 2, 4, 8):
        s0 = oracle.scores(np.zeros((1, 16)), "softmax")
        ids0, _ = oracle.select_topk(s0, K)
        assert list(ids0[0]) == list(range(K))
        assert np.all(oracle.topk_weights(s0, ids0, True, 1.0) == 1.0 / K)


def test_no_renorm_weight_is_the_softmax_probability():
    cfg = get_config("dspark", T=64)
    inp = make_inputs(cfg)
    res = oracle_forward(inp)
    p = torch.softmax(torch.from_numpy(res.logits), dim=1).numpy()
    np.testing.assert_allclose(res.weights[:, 0], np.take_along_axis(p, res.ids, 1)[:, 0], rtol=1e-13)
    assert np.all(res.weights < 1.0)
    # the bias moved the choice but not the weight
    assert not np.array_equal(np.argmax(res.scores, axis=1), res.ids[:, 0])


def test_route_is_the_routing_half_of_forward():
    from dataclasses import replace
    # the tiny layer (softmax, ties) and a reduced DSV4-like one (sigmoid, bias, route_scale 2.5)
    for cfg in (get_config("tiny"), replace(get_config("dsv4", T=64), D=256, I=64, Is=0)):
        inp = make_inputs(cfg)
        full = oracle_forward(inp)
        rt = oracle.route(inp.x, inp.w_router, K=cfg.K, score=cfg.score, renorm=cfg.renorm,
                          route_scale=cfg.route_scale, bias=inp.bias)
        for f in ("logits", "scores", "choice", "ids", "weights", "rel_margin", "exempt"):
            assert np.array_equal(getattr(rt, f), getattr(full, f)), (cfg.name, f)


# ---------------------------------------------------------------- dispatch

def test_permutation_matches_stable_argsort_and_invariants():
    rng = np.random.default_rng(17)
    T, E, K = 777, 37, 5
    ids = np.sort(np.stack([rng.choice(E, K, replace=False) for _ in range(T)]), axis=1).astype(np.int32)
    masked = rng.random(T) < 0.1
    ids[masked] = -1
    pm = oracle.permute(ids, E)
    t_of = np.repeat(np.arange(T), K)
    e_of = ids.reshape(-1)
    keep = e_of >= 0
    order = np.argsort(e_of[keep].astype(np.int64) * T + t_of[keep], kind="stable")
    np.testing.assert_array_equal(pm["perm_token"], t_of[keep][order])
    np.testing.assert_array_equal(pm["counts"], np.bincount(e_of[keep], minlength=E))
    assert pm["offsets"][0] == 0 and pm["offsets"][E] == keep.sum()
    inv = pm["inv_pos"]
    assert np.all(inv[masked] == -1)
    pos = inv[~masked].reshape(-1)
    assert sorted(pos.tolist()) == list(range(keep.sum()))      # bijection
    for t in np.nonzero(~masked)[0][:200]:
        for j in range(K):
            assert pm["perm_token"][inv[t, j]] == t
            e = ids[t, j]
            assert pm["offsets"][e] <= inv[t, j] < pm["offsets"][e + 1]
    for e in range(E):
        seg = pm["perm_token"][pm["offsets"][e]:pm["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)


# ---------------------------------------------------------------- expert MLP

def _torch_swiglu(x, w1, w2):
    I = w2.shape[1]
    h = x @ w1.T
    return (torch.nn.functional.silu(h[:, :I]) * h[:, I:]) @ w2.T


def test_layer_matches_dense_all_experts_formulation():
    cfg = get_config("tiny")
    inp = make_inputs(cfg)
    res = oracle_forward(inp)
    x = torch.from_numpy(oracle.widen(inp.x))
    gate = torch.zeros(cfg.T, cfg.E, dtype=torch.float64)
    for t in range(cfg.T):
        for j in range(cfg.K):
            gate[t, res.ids[t, j]] = res.weights[t, j]
    dense = torch.zeros(cfg.T, cfg.D, dtype=torch.float64)
    for e in range(cfg.E):
        ye = _torch_swiglu(x, torch.from_numpy(oracle.widen(inp.w_gate_up[e])),
                           torch.from_numpy(oracle.widen(inp.w_down[e])))
        dense += gate[:, e:e + 1] * ye
    rms = float(torch.sqrt(torch.mean(dense ** 2)))
    assert float(torch.max(torch.abs(dense - torch.from_numpy(res.out)))) <= 1e-12 * rms


def test_single_expert_top1_is_a_dense_swiglu_mlp():
    rng = np.random.default_rng(18)
    T, D, I = 40, 64, 96
    x = rng.standard_normal((T, D)).astype(np.float32)
    wr = rng.standard_normal((1, D)).astype(np.float32)
    w1 = (rng.standard_normal((1, 2 * I, D)) * 0.1).astype(np.float32)
    w2 = (rng.standard_normal((1, D, I)) * 0.1).astype(np.float32)
    res = oracle.forward(x, wr, w1, w2, K=1, score="softmax", renorm=True, route_scale=1.0,
                         bf16_mode=False)
    assert np.all(res.weights == 1.0)
    ref = _torch_swiglu(torch.from_numpy(x.astype(np.float64)), torch.from_numpy(w1[0].astype(np.float64)),
                        torch.from_numpy(w2[0].astype(np.float64))).numpy()
    np.testing.assert_allclose(res.out, ref, rtol=1e-12, atol=1e-14)


def test_shared_expert_added_on_every_kept_token():
    cfg = get_config("tiny")
    inp = make_inputs(cfg)
    rng = np.random.default_rng(19)
    w1s = (rng.standard_normal((2 * 64, cfg.D)) * 0.02).astype(np.float32)
    w2s = (rng.standard_normal((cfg.D, 64)) * 0.02).astype(np.float32)
    mask = np.ones(cfg.T, dtype=np.uint8)
    mask[[3, 9]] = 0
    base = oracle_forward(inp, mask=mask)
    inp.w_gate_up_s, inp.w_down_s = w1s, w2s
    with_s = oracle_forward(inp, mask=mask)
    sh = _torch_swiglu(torch.from_numpy(oracle.widen(inp.x)), torch.from_numpy(w1s.astype(np.float64)),
                       torch.from_numpy(w2s.astype(np.float64))).numpy()
    sh[[3, 9]] = 0.0
    np.testing.assert_allclose(with_s.out - base.out, sh, rtol=1e-10, atol=1e-15)
    assert np.all(with_s.out[[3, 9]] == 0.0)
    assert np.all(with_s.ids[[3, 9]] == -1) and with_s.offsets[-1] == (cfg.T - 2) * cfg.K


def test_bf16_mode_rounds_activation_and_output():
    cfg = get_config("dspark", T=16)
    inp = make_inputs(cfg)
    res = oracle_forward(inp)
    assert np.array_equal(oracle.round_bf16(res.y), res.y)      # expert outputs on the bf16 grid
    assert np.array_equal(oracle.round_bf16(res.y_exact), res.y)
    assert not np.array_equal(res.y_exact, res.y)
    # the reference output is built from the exact expert outputs
    ref = np.zeros_like(res.out)
    for j in range(cfg.K):
        ref += res.weights[:, j:j + 1] * res.y_exact[res.inv_pos[:, j]]
    np.testing.assert_array_equal(res.out, ref)
    # the activation is a bf16 operand: one expert recomputed with torch, a rounded by torch's cast
    e = int(res.ids[0, 0])
    rows = res.perm_token[res.offsets[e]:res.offsets[e + 1]]
    x = torch.from_numpy(oracle.widen(inp.x[rows]))
    w1 = torch.from_numpy(oracle.widen(inp.w_gate_up[e]))
    w2 = torch.from_numpy(oracle.widen(inp.w_down[e]))
    I = cfg.I
    h = (x @ w1.T).numpy()
    a64 = oracle.silu(h[:, :I]) * h[:, I:]
    # torch's cast goes through float32, so it may differ from the single rounding on the
    # rare values that round twice; everywhere else the two agree
    a_bf = torch.from_numpy(a64).float().to(torch.bfloat16).double().numpy()
    assert np.mean(a_bf == oracle.round_bf16(a64)) > 0.999
    y_ref = (torch.from_numpy(oracle.round_bf16(a64)) @ w2.T).numpy()
    np.testing.assert_allclose(res.y_exact[res.offsets[e]:res.offsets[e + 1]], y_ref, rtol=1e-12, atol=1e-18)


# ---------------------------------------------------------------- combine

def test_combine_matches_exact_rational_per_operation():
    rng = np.random.default_rng(20)
    T, K, D = 5, 6, 24
    y = oracle.bf16_bits_of(rng.standard_normal((T * K, D)).astype(np.float32))
    inv = rng.permutation(T * K).reshape(T, K).astype(np.int32)
    w = rng.uniform(0.0, 1.0, (T, K)).astype(np.float32)
    sh = oracle.bf16_bits_of(rng.standard_normal((T, D)).astype(np.float32))
    got32 = oracle.combine_fp32(y, inv, w, sh, out="f32")
    gotbf = oracle.combine_fp32(y, inv, w, sh, out="bf16")
    yf = oracle.widen(y)
    sf = oracle.widen(sh)
    for t in range(T):
        for d in range(D):
            acc = Fraction(0)
            for j in range(K):
                p = _r32(Fraction(float(w[t, j])) * Fraction(float(yf[inv[t, j], d])))
                acc = _r32(acc + p)
            acc = _r32(acc + Fraction(float(sf[t, d])))
            assert Fraction(float(got32[t, d])) == acc
            bf = (np.uint32(gotbf[t, d]) << np.uint32(16)).view(np.float32)
            assert Fraction(float(bf)) == _rbf16(acc)


def test_combine_is_the_sum_of_weighted_terms_within_fold_bound():
    rng = np.random.default_rng(21)
    T, K, D = 64, 6, 256
    y = oracle.bf16_bits_of(rng.standard_normal((T * K, D)).astype(np.float32))
    inv = np.arange(T * K, dtype=np.int32).reshape(T, K)
    w = rng.uniform(0, 1, (T, K)).astype(np.float32)
    got = oracle.combine_fp32(y, inv, w, out="f32").astype(np.float64)
    terms = w.astype(np.float64)[:, :, None] * oracle.widen(y)[inv]
    exact = terms.sum(axis=1)
    u = 2.0 ** -24
    bound = (2 * K) * u * np.abs(terms).sum(axis=1)   # K products and K sums, first order
    assert np.all(np.abs(got - exact) <= bound * 1.01)


def test_combine_top1_unit_weight_is_identity():
    rng = np.random.default_rng(22)
    y = rng.standard_normal((10, 32)).astype(np.float32)
    inv = np.arange(10, dtype=np.int32).reshape(10, 1)
    out = oracle.combine_fp32(y, inv, np.ones((10, 1), np.float32), out="f32")
    assert np.array_equal(out.view(np.uint32), y.view(np.uint32))


def test_combine_720_orders_give_360_classes_as_printed():
    with open(os.path.join(GOLDEN, "arxiv_2607_28097_reduction_orders.json")) as f:
        g = json.load(f)
    K = g["routed_terms"]
    rng = np.random.default_rng(23)
    T, D = 6, 256
    y = oracle.bf16_bits_of((rng.standard_normal((T * K, D)) * 0.3).astype(np.float32))
    inv = rng.permutation(T * K).reshape(T, K).astype(np.int32)
    # weights of comparable size, as renormalised routing weights are (a term far below
    # the others can make some orders coincide on every element, giving fewer classes)
    w = rng.uniform(0.5, 1.5, (T, K))
    w = (w / w.sum(axis=1, keepdims=True) * 2.5).astype(np.float32)
    res = oracle.combine_orders(y, inv, w)
    assert len(res) == g["orders"]
    ident = tuple(range(K))
    swap01 = (1, 0) + tuple(range(2, K))
    for pi, r in res.items():
        pj = (pi[1], pi[0]) + pi[2:]
        assert np.array_equal(r.view(np.uint32), res[pj].view(np.uint32))
    for t in range(T):
        classes = {res[pi][t].tobytes() for pi in res}
        assert len(classes) == g["b_mode_exact_structural_classes"]
        canon = res[ident][t].tobytes()
        same = {pi for pi in res if res[pi][t].tobytes() == canon}
        assert same == {ident, swap01}
    # the canonical order is the default combine
    assert np.array_equal(res[ident], oracle.combine_fp32(y, inv, w, out="f32"))


# ------------------------------------------------- order-invariant combine

def test_combine_f64_is_the_exact_sum_rounded_once():
    rng = np.random.default_rng(24)
    T, K, D = 5, 6, 24
    y = oracle.bf16_bits_of(rng.standard_normal((T * K, D)).astype(np.float32))
    inv = rng.permutation(T * K).reshape(T, K).astype(np.int32)
    w = rng.uniform(0.0, 1.0, (T, K)).astype(np.float32)
    sh = oracle.bf16_bits_of(rng.standard_normal((T, D)).astype(np.float32))
    got32 = oracle.combine_f64(y, inv, w, sh, out="f32")
    gotbf = oracle.combine_f64(y, inv, w, sh, out="bf16")
    yf = oracle.widen(y)
    sf = oracle.widen(sh)
    for t in range(T):
        for d in range(D):
            exact = sum(Fraction(float(w[t, j])) * Fraction(float(yf[inv[t, j], d])) for j in range(K))
            exact += Fraction(float(sf[t, d]))
            assert Fraction(float(got32[t, d])) == _r32(exact)
            bf = (np.uint32(gotbf[t, d]) << np.uint32(16)).view(np.float32)
            assert Fraction(float(bf)) == _rbf16(exact)


def test_combine_f64_all_720_orders_agree():
    rng = np.random.default_rng(25)
    K, T, D = 6, 6, 256
    y = oracle.bf16_bits_of((rng.standard_normal((T * K, D)) * 0.3).astype(np.float32))
    inv = rng.permutation(T * K).reshape(T, K).astype(np.int32)
    w = rng.uniform(0.5, 1.5, (T, K))
    w = (w / w.sum(axis=1, keepdims=True) * 2.5).astype(np.float32)
    res = oracle.combine_orders(y, inv, w, mode="f64")
    assert len(res) == 720
    first = next(iter(res.values())).view(np.uint32)
    for r in res.values():
        assert np.array_equal(r.view(np.uint32), first)
    # while the float32 fold of the same terms splits into 360 classes per token
    res32 = oracle.combine_orders(y, inv, w, mode="f32")
    assert all(len({res32[pi][t].tobytes() for pi in res32}) == 360 for t in range(T))


def test_combine_f64_masked_and_unit_weight():
    rng = np.random.default_rng(26)
    y = rng.standard_normal((10, 32)).astype(np.float32)
    inv = np.arange(10, dtype=np.int32).reshape(10, 1)
    out = oracle.combine_f64(y, inv, np.ones((10, 1), np.float32), out="f32")
    assert np.array_equal(out.view(np.uint32), y.view(np.uint32))
    inv[3, 0] = -1
    out = oracle.combine_f64(y, inv, np.ones((10, 1), np.float32), out="f32")
    assert np.all(out[3] == 0)


# ---------------------------------------------------------------- backward

class _RoundGrad(torch.autograd.Function):
    """Identity whose backward rounds the incoming gradient to bf16."""

    @staticmethod
    def forward(ctx, v):
        return v.view_as(v)

    @staticmethod
    def backward(ctx, g):
        return torch.from_numpy(oracle.round_bf16(g.detach().numpy()))


def _autograd_grads(x, wr, w1, w2, w1s, w2s, ids, G, score, renorm, rs, mask, bf16_mode, grad_bf16=False):
    """An independently written forward in float64 torch, differentiated by
    autograd; bf16 rounding points pass the gradient straight through.  With
    grad_bf16 the gradients arriving at the logits, at each expert's gate/up
    projection and at each routed expert output are rounded to bf16."""
    F = torch.nn.functional
    gr = _RoundGrad.apply if grad_bf16 else (lambda v: v)
    tt = lambda a: torch.tensor(oracle.widen(a), dtype=torch.float64, requires_grad=True)
    X, Wr, W1, W2 = tt(x), tt(wr), tt(w1), tt(w2)
    W1s = tt(w1s) if w1s is not None else None
    W2s = tt(w2s) if w2s is not None else None

    def rnd(v):
        if not bf16_mode:
            return v
        r = torch.from_numpy(oracle.round_bf16(v.detach().numpy()))
        return v + (r - v).detach()

    logits = gr(X @ Wr.T)
    if score == "softmax":
        s = torch.softmax(logits, dim=1)
    elif score == "sigmoid":
        s = torch.sigmoid(logits)
    else:
        s = torch.sqrt(F.softplus(logits))
    T, K = ids.shape
    I = w2.shape[2]
    out = []
    for t in range(T):
        if mask is not None and not mask[t]:
            out.append(torch.zeros(X.shape[1], dtype=torch.float64))
            continue
        sel = torch.stack([s[t, int(e)] for e in ids[t]])
        w = sel / sel.sum() * rs if renorm else sel * rs
        o = 0.0
        for j, e in enumerate(ids[t]):
            h = gr(W1[int(e)] @ X[t])
            a = rnd(F.silu(h[:I]) * h[I:])
            o = o + w[j] * gr(rnd(W2[int(e)] @ a))
        if W1s is not None:
            Is = w2s.shape[1]
            hs = gr(W1s @ X[t])
            o = o + rnd(W2s @ rnd(F.silu(hs[:Is]) * hs[Is:]))
        out.append(o)
    loss = (torch.stack(out) * torch.from_numpy(oracle.widen(G))).sum()
    loss.backward()
    g = {"dx": X.grad, "d_router": Wr.grad, "d_gate_up": W1.grad, "d_down": W2.grad}
    if W1s is not None:
        g.update({"d_gate_up_shared": W1s.grad, "d_down_shared": W2s.grad})
    return {k: v.numpy() for k, v in g.items()}


@pytest.mark.parametrize("score,renorm,bf16,shared,masked,grad_bf16", [
    ("softmax", True, False, False, False, False),
    ("sigmoid", True, True, True, True, False),
    ("sqrtsoftplus", False, False, True, False, False),
    ("sigmoid", False, True, False, True, False),
    ("sqrtsoftplus", True, True, True, True, False),
    ("softmax", True, True, True, False, True),
    ("sigmoid", True, True, True, True, True),
    ("sqrtsoftplus", False, True, False, False, True),
])
def test_backward_matches_torch_autograd(score, renorm, bf16, shared, masked, grad_bf16):
    rng = np.random.default_rng(31)
    T, D, E, K, I, Is = 12, 32, 8, 3, 16, 16
    f = (lambda a: oracle.round_bf16(a)) if bf16 else (lambda a: a)
    x = f(rng.standard_normal((T, D)))
    wr = f(rng.standard_normal((E, D)) * 0.3)
    w1 = f(rng.standard_normal((E, 2 * I, D)) * 0.2)
    w2 = f(rng.standard_normal((E, D, I)) * 0.2)
    w1s = f(rng.standard_normal((2 * Is, D)) * 0.2) if shared else None
    w2s = f(rng.standard_normal((D, Is)) * 0.2) if shared else None
    G = f(rng.standard_normal((T, D)))
    mask = (rng.random(T) > 0.25).astype(np.uint8) if masked else None
    bias = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    fw = oracle.forward(x, wr, w1, w2, K=K, score=score, renorm=renorm, route_scale=1.5, bias=bias, mask=mask,
                        shared_gate_up=w1s, shared_down=w2s, bf16_mode=bf16)
    got = oracle.backward(x, wr, w1, w2, G, fw.ids, score=score, renorm=renorm, route_scale=1.5, mask=mask,
                          shared_gate_up=w1s, shared_down=w2s, bf16_mode=bf16, grad_bf16=grad_bf16)
    ids_full = np.where(fw.ids >= 0, fw.ids, 0)
    ref = _autograd_grads(x, wr, w1, w2, w1s, w2s, ids_full, G, score, renorm, 1.5,
                          None if mask is None else mask.astype(bool), bf16, grad_bf16)
    for k, v in ref.items():
        scale = max(1e-300, float(np.abs(v).max()))
        assert np.max(np.abs(got[k] - v)) <= 1e-11 * scale, k
    if mask is not None:
        assert np.all(got["dx"][~mask.astype(bool)] == 0)
    if grad_bf16:  # the rounding is exercised: the exact gradients differ
        exact = oracle.backward(x, wr, w1, w2, G, fw.ids, score=score, renorm=renorm, route_scale=1.5, mask=mask,
                                shared_gate_up=w1s, shared_down=w2s, bf16_mode=bf16)
        for k in ("dx", "d_router", "d_gate_up", "d_down"):
            assert not np.array_equal(exact[k], got[k]), k
    # the weight gradient dw is the inner product of G with the bf16 expert output the combine used
    t, j = np.argwhere(fw.ids >= 0)[0]
    p = fw.inv_pos[t, j]
    assert abs(got["dw"][t, j] - float(np.dot(oracle.widen(G)[t], fw.y[p]))) <= 1e-12 * (1 + abs(got["dw"][t, j]))


def test_backward_of_unpicked_expert_is_zero():
    rng = np.random.default_rng(32)
    T, D, E, K, I = 6, 16, 8, 1, 8
    x = rng.standard_normal((T, D))
    wr = rng.standard_normal((E, D))
    w1 = rng.standard_normal((E, 2 * I, D))
    w2 = rng.standard_normal((E, D, I))
    ids = np.array([[0], [0], [1], [1], [2], [0]], dtype=np.int32)
    g = oracle.backward(x, wr, w1, w2, rng.standard_normal((T, D)), ids, score="sigmoid", renorm=False,
                        route_scale=1.0, bf16_mode=False)
    assert np.all(g["d_gate_up"][3:] == 0) and np.all(g["d_down"][3:] == 0)
    # sigmoid scores: only the picked experts' logits receive a gradient
    picked = np.zeros((T, E), bool)
    picked[np.arange(T), ids[:, 0]] = True
    assert np.all(g["dlogits"][~picked] == 0) and np.all(g["dlogits"][picked] != 0)


def test_backward_expert_equals_the_full_backward():
    """The one-expert entry takes the same steps as the full backward."""
    rng = np.random.default_rng(33)
    T, D, E, K, I = 20, 32, 8, 3, 16
    r = oracle.round_bf16
    x, wr = r(rng.standard_normal((T, D))), r(rng.standard_normal((E, D)) * 0.3)
    w1, w2 = r(rng.standard_normal((E, 2 * I, D)) * 0.2), r(rng.standard_normal((E, D, I)) * 0.2)
    G = r(rng.standard_normal((T, D)))
    mask = (rng.random(T) > 0.2).astype(np.uint8)
    for score, renorm, gb in (("sigmoid", True, True), ("softmax", False, False)):
        fw = oracle.forward(x, wr, w1, w2, K=K, score=score, renorm=renorm, route_scale=2.0, mask=mask,
                            bf16_mode=True)
        full = oracle.backward(x, wr, w1, w2, G, fw.ids, score=score, renorm=renorm, route_scale=2.0, mask=mask,
                               bf16_mode=True, grad_bf16=gb)
        for e in range(E):
            d1, d2 = oracle.backward_expert(e, x, wr, w1[e], w2[e], G, fw.ids, score=score, renorm=renorm,
                                            route_scale=2.0, mask=mask, bf16_mode=True, grad_bf16=gb)
            assert np.array_equal(d1, full["d_gate_up"][e]) and np.array_equal(d2, full["d_down"][e]), e
