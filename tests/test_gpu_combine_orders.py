"""Reduction-order check of the combine on a DeepSeek-V4-Flash-like layer.

arXiv 2607.28097 ("From Expert Reduction to Behavioral Divergence", Abstract)
aggregates the six routed expert terms of a DeepSeek-V4-Flash layer in all
720 orders and finds 360 exact classes in its B mode.  Here the GPU's own six
weighted expert outputs of 1024 tokens are folded in every order by the
float32 emulation: the GPU result must be the canonical (ascending expert id)
class and no other, and no token may show more than 360 classes.  Two operand
modes: bf16 expert outputs from the bf16-operand forward, and float32 expert
outputs from a float32-operand forward of the same tokens (the same bf16
values widened exactly).
"""

import itertools
import json

import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs
from tests.gpu_util import make_layer, to_dev, to_host

pytestmark = pytest.mark.gpu

NTOK = 1024


@pytest.fixture(scope="module")
def dsv4():
    cfg = get_config("dsv4", T=NTOK)
    print(f"[orders] drawing DSV4-like inputs (T={NTOK})", flush=True)
    return make_inputs(cfg)


def _layer_f32(layer_bf16):
    from routing_grouped_gemm_gemv_amd import MoeLayer
    s = layer_bf16.shape.replace(dtype="f32")
    W = {k: v.float() for k, v in layer_bf16.weights.items()}
    return MoeLayer(s, W["router"], W["gate_up"], W["down"], W.get("gate_up_shared"), W.get("down_shared"),
                    layer_bf16.sel_bias)


@pytest.mark.parametrize("mode", ["bf16", "f32"])
def test_combine_is_the_canonical_order_of_720(dsv4, mode):
    from routing_grouped_gemm_gemv_amd import binding as B
    layer = make_layer(dsv4)
    x = to_dev(dsv4.x)
    if mode == "f32":
        layer = _layer_f32(layer)
        x = x.float()
    _, tr = layer.forward(x, trace=True)
    out32 = torch.empty(NTOK, layer.shape.D, dtype=torch.float32, device="cuda")
    B.moe_combine(layer.with_tokens(NTOK), tr["y"], tr["inv_pos"], tr["topk_w"], tr["shared_out"], out32)
    torch.cuda.synchronize()
    y = to_host(tr["y"])
    inv = to_host(tr["inv_pos"])
    w = to_host(tr["topk_w"])
    sh = to_host(tr["shared_out"])
    g = to_host(out32)
    K = inv.shape[1]
    assert K == 6
    ident = tuple(range(K))
    swap01 = (1, 0) + tuple(range(2, K))
    match_all = None
    classes = [set() for _ in range(NTOK)]
    n_orders = 0
    for pi in itertools.permutations(range(K)):
        r = oracle.combine_fp32(y, inv, w, sh, order=pi, out="f32")
        eq = np.all(r.view(np.uint32) == g.view(np.uint32), axis=1)
        if pi == ident:
            assert eq.all(), "GPU combine differs from the ascending-id fold"
        if eq.all():
            match_all = (match_all or set()) | {pi}
        for t in range(NTOK):
            classes[t].add(hash(r[t].tobytes()))
        n_orders += 1
    assert n_orders == 720
    assert match_all == {ident, swap01}, match_all
    ncls = np.array([len(c) for c in classes])
    print(f"[orders] {mode}: " + json.dumps({"orders": n_orders, "max_classes": int(ncls.max()),
                                               "tokens_with_360": int((ncls == 360).sum()),
                                               "min_classes": int(ncls.min())}), flush=True)
    assert ncls.max() <= 360


@pytest.mark.parametrize("mode", ["bf16", "f32"])
def test_order_invariant_combine_is_every_order(dsv4, mode):
    """The float64 combine mode on the same expert outputs: bit-equal to the
    oracle's float64 sum rounded once, and every one of the 720 orders of the
    six routed terms gives that same result."""
    from routing_grouped_gemm_gemv_amd import binding as B
    layer = make_layer(dsv4)
    x = to_dev(dsv4.x)
    if mode == "f32":
        layer = _layer_f32(layer)
        x = x.float()
    _, tr = layer.forward(x, trace=True)
    shape = layer.with_tokens(NTOK).replace(combine="f64")
    out32 = torch.empty(NTOK, layer.shape.D, dtype=torch.float32, device="cuda")
    outbf = torch.empty(NTOK, layer.shape.D, dtype=torch.bfloat16, device="cuda")
    B.moe_combine(shape, tr["y"], tr["inv_pos"], tr["topk_w"], tr["shared_out"], out32)
    B.moe_combine(shape, tr["y"], tr["inv_pos"], tr["topk_w"], tr["shared_out"], outbf)
    torch.cuda.synchronize()
    y, inv, w, sh = (to_host(tr[k]) for k in ("y", "inv_pos", "topk_w", "shared_out"))
    g32 = to_host(out32)
    gbf = to_host(outbf)
    assert np.array_equal(gbf, oracle.combine_f64(y, inv, w, sh, out="bf16"))
    for pi in itertools.permutations(range(inv.shape[1])):
        r = oracle.combine_f64(y, inv, w, sh, order=pi, out="f32")
        assert np.array_equal(r.view(np.uint32), g32.view(np.uint32)), pi
    print(f"[orders] f64 combine, {mode} operands: all 720 orders equal the GPU result", flush=True)
