"""Routing variants against the CPU oracle, through the C ABI.

The SpecForge pull request #1003 commit notes name two routing variants
without formulas: sqrtsoftplus routers (notes on the load-balance loss) and
DeepSeek-V3's group-limited select (notes on select).  Readings: the score is
sqrt(log(1 + e^l)); experts form n_group groups of consecutive ids, a group's
score is the sum of its two largest choices, the topk_group best groups are
kept (ties to the lower group id) and the K experts are chosen among them.

Routing acceptance as for the plain router: ids bit-exact except tokens the
oracle marks as near ties (the margin of a grouped token also covers the
group decision), weights within 2e-6 relative, float32 logits within 2e-6.
The layer tests run the full acceptance of test_gpu_parity on the variants.
"""

import json
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs
from synth.gen import hidden_states, router_weights, selection_bias
from tests.gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


ROUTE_CASES = [
    # config, T, score, n_group, topk_group
    ("dsv4", 32768, "sqrtsoftplus", 1, 1),   # fused kernel, 128-token tiles
    ("dsv4", 2048, "sqrtsoftplus", 1, 1),    # fused kernel, 64-token tiles
    ("dsv4", 2048, "sigmoid", 8, 4),         # DeepSeek-V3-like grouping, selection bias
    ("dsv4", 2048, "sqrtsoftplus", 8, 4),
    ("dsv4", 1000, "sigmoid", 64, 2),        # 64 groups of 4, two kept
    ("dsv4", 64, "sigmoid", 64, 1),          # K = 6 > the 4 experts of one group: rejected
    ("q30", 1024, "softmax", 8, 4),
    ("q30", 1024, "sqrtsoftplus", 16, 3),
    ("qnext", 512, "softmax", 8, 2),         # E = 512: eight experts per lane in the wave top-k
    ("qnext", 512, "sqrtsoftplus", 1, 1),
    ("dspark", 1024, "sqrtsoftplus", 4, 2),  # E = 8, top-1, no renorm, selection bias
    ("tiny", 64, "sqrtsoftplus", 2, 1),      # fp32 operands
]


def _route(cfg):
    from routing_grouped_gemm_gemv_amd import binding as B
    T = cfg.T
    x = hidden_states(cfg, T)
    wr = router_weights(cfg)
    bias = selection_bias(cfg)
    shape = B.Shape(T=T, D=cfg.D, E=cfg.E, K=cfg.K, I=cfg.I, Is=cfg.Is, score=cfg.score, renorm=cfg.renorm,
                    route_scale=cfg.route_scale, dtype=cfg.dtype, n_group=cfg.n_group,
                    topk_group=cfg.topk_group)
    ws = B.alloc_workspace(shape)
    logits = torch.empty(T, cfg.E, dtype=torch.float32, device="cuda")
    ids = torch.full((T, cfg.K), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, cfg.K), -7.0, dtype=torch.float32, device="cuda")
    B.moe_route(shape, to_dev(x), to_dev(wr), to_dev(bias), None, logits, ids, w, ws)
    torch.cuda.synchronize()
    return x, wr, bias, to_host(logits), to_host(ids), to_host(w)


def _oracle_route(cfg, x, wr, bias):
    lg = oracle.router_logits(oracle.widen(x), oracle.widen(wr))
    s = oracle.scores(lg, cfg.score)
    c = s + oracle.widen(bias)[None, :] if bias is not None else s
    if cfg.n_group > 1:
        ids, margin = oracle.select_grouped(c, cfg.K, cfg.n_group, cfg.topk_group)
    else:
        ids, margin = oracle.select_topk(c, cfg.K)
    return lg, ids, margin, s


@pytest.mark.parametrize("name,T,score,G,TG", ROUTE_CASES)
def test_route_variant(name, T, score, G, TG):
    cfg = get_config(name, T=T, score=score, n_group=G, topk_group=TG)
    if G > 1 and cfg.K > TG * (cfg.E // G):
        from routing_grouped_gemm_gemv_amd import binding as B
        with pytest.raises(B.MoeError):
            _route(cfg)
        return
    _say(f"[variants] route {name} T={T} score={score} n_group={G} topk_group={TG}")
    x, wr, bias, glog, gids, gw = _route(cfg)
    lg, ids, margin, s = _oracle_route(cfg, x, wr, bias)
    exempt = (margin > 0) & (margin < oracle.EXEMPT_REL_MARGIN)
    same = np.all(gids == ids, axis=1)
    bad = np.nonzero(~same & ~exempt)[0]
    rep = {"tokens": T, "exempt": int(exempt.sum()), "exempt_differing": int((~same & exempt).sum()),
           "mismatch": int(bad.size), "mismatch_tokens": bad[:10].tolist()}
    _say(f"[variants] {json.dumps(rep)}")
    assert bad.size == 0, rep
    w_ref = oracle.topk_weights(s, ids, cfg.renorm, cfg.route_scale)
    np.testing.assert_allclose(gw[same], w_ref[same], rtol=2e-6, atol=1e-7)
    assert np.max(np.abs(glog - lg) / np.maximum(1.0, np.abs(lg))) < 2e-6
    if G > 1:
        gs = cfg.E // G
        # every pick lies in one of topk_group groups
        assert all(len(set((gids[t] // gs).tolist())) <= TG for t in range(T))


LAYER_CASES = [
    ("tiny", None, "sqrtsoftplus", 4, 2),
    ("tiny", None, "sigmoid", 2, 1),
    ("q30", 256, "sqrtsoftplus", 8, 4),
    ("q30", 256, "softmax", 16, 2),
]


@pytest.mark.parametrize("name,T,score,G,TG", LAYER_CASES)
def test_layer_variant(name, T, score, G, TG):
    from tests.test_gpu_parity import check_layer
    cfg = get_config(name, T=T, score=score, n_group=G, topk_group=TG)
    check_layer(make_inputs(cfg), label=f"{name}-{score}-g{G}k{TG}")
