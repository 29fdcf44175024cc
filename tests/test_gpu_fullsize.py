"""Parity at the workloads' full sizes, in the launch configuration the benchmark
times (moe_forward over the whole batch, bf16 output).

Over every token: the top-k ids against the oracle's router (bit-exact except
near ties at the K boundary, which are counted and reported: RL-Kernel roadmap,
"Problem 1: Routing Is A Discrete Decision", any mismatch is reported), the
weights, the permutation of the GPU's ids, and the combine bit for bit against
the oracle's float32 fold of the GPU's own expert outputs.  The expert MLPs
(the oracle's float64 matmuls) run on sampled tokens, since a token's output
depends on that token alone (the invariance tests show it).
"""

import json

import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs
from tests.gpu_util import check_layer_output, make_layer, routing_check, to_dev, to_host
from tests.oracle_bridge import oracle_forward

pytestmark = pytest.mark.gpu

SAMPLES = {"dsv4": 48, "qnext": 96, "q30": 128, "dspark": 128}
TOL = 2e-2


@pytest.mark.parametrize("name", ["dspark", "q30", "qnext", "dsv4"])
def test_full_size_layer(name):
    cfg = get_config(name)
    print(f"[fullsize] {name} T={cfg.T}: drawing inputs", flush=True)
    inp = make_inputs(cfg)
    layer = make_layer(inp)
    x = to_dev(inp.x)
    out, tr = layer.forward(x, trace=True)
    torch.cuda.synchronize()
    print(f"[fullsize] {name}: forward done", flush=True)
    ids = to_host(tr["topk_ids"])
    inv = to_host(tr["inv_pos"])
    w = to_host(tr["topk_w"])
    gout = to_host(out)

    # (a) routing of every token against the oracle's router
    rt = oracle.route(inp.x, inp.w_router, K=cfg.K, score=cfg.score, renorm=cfg.renorm,
                      route_scale=cfg.route_scale, bias=inp.bias, n_group=cfg.n_group, topk_group=cfg.topk_group)
    rc = routing_check(ids, rt)
    print(f"[fullsize] {name} routing over all {cfg.T} tokens: {json.dumps(rc)}", flush=True)
    assert rc["mismatch_count"] == 0, rc
    same = np.all(ids == rt.ids, axis=1)
    np.testing.assert_allclose(w[same], rt.weights[same], rtol=2e-6, atol=1e-7)

    # (a) dispatch of the GPU's ids, all T*K pairs
    pm = oracle.permute(ids, cfg.E)
    np.testing.assert_array_equal(to_host(tr["counts"]), pm["counts"])
    np.testing.assert_array_equal(to_host(tr["offsets"]), pm["offsets"])
    nv = int(pm["offsets"][-1])
    np.testing.assert_array_equal(to_host(tr["perm_token"])[:nv], pm["perm_token"])
    np.testing.assert_array_equal(inv, pm["inv_pos"])

    # (b) the combine of every token on the GPU's own expert outputs
    y = to_host(tr["y"])[:nv]
    sh = to_host(tr["shared_out"]) if cfg.Is else None
    emu = oracle.combine_fp32(y, inv, w, sh, out="bf16")
    nbad = int(np.sum(np.any(gout != emu, axis=1)))
    assert nbad == 0, f"combine differs from the float32 fold on {nbad} of {cfg.T} tokens"
    del y, emu

    # (c) sampled tokens through the oracle's expert MLPs
    rng = np.random.default_rng(1234)
    tok = np.sort(rng.choice(cfg.T, SAMPLES[name], replace=False))
    ref = oracle_forward(inp, tokens=tok)
    assert np.array_equal(ref.ids, rt.ids[tok])
    ref_out = ref.out.copy()
    diff = np.nonzero(~same[tok])[0]
    if diff.size:
        rep = oracle_forward(inp, tokens=tok, ids_override=ids[tok])
        ref_out[diff] = rep.out[diff]
    counts = pm["counts"]
    info = {"exempt_count": rc["exempt_count"], "exempt_differing": rc["exempt_differing"],
            "mismatch_count": rc["mismatch_count"], "load_max_over_mean": float(counts.max() / counts.mean()),
            "empty_experts": int((counts == 0).sum())}
    pr = check_layer_output(layer.with_tokens(cfg.T), tr, gout, ref_out, None, TOL, info, tokens=tok)
    print(f"[fullsize] {name} {json.dumps(pr)}", flush=True)
