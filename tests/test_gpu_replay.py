"""Routing replay (moe_forward_replay) against the oracle's replay.

The RL-Kernel roadmap ("R3 Should Not Be A Prerequisite") replays the experts
a token used in another run while the router still scores them.  Checks: a
replay of the layer's own ids reproduces its output bit for bit; a replay of
different ids (each token's K-th expert swapped for its (K+1)-th) matches the
oracle run with the same ids; tokens with invalid replayed ids are masked.
"""

import functools
import json
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs
from tests.gpu_util import check_layer_output, make_layer, to_dev, to_host
from tests.oracle_bridge import oracle_forward

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def _inputs(name, T):
    _say(f"[replay] drawing {name} inputs (T={T})")
    return make_inputs(get_config(name, T=T))


@pytest.mark.parametrize("name,T", [("dsv4", 300), ("qnext", 200)])
def test_replay_of_own_ids_reproduces_the_forward(name, T):
    inp = _inputs(name, T)
    layer = make_layer(inp)
    x = to_dev(inp.x)
    out, tr = layer.forward(x, trace=True)
    out2, tr2 = layer.forward(x, trace=True, replay_ids=tr["topk_ids"].clone())
    torch.cuda.synchronize()
    assert torch.equal(tr["topk_ids"], tr2["topk_ids"])
    assert torch.equal(tr["topk_w"].view(torch.int32), tr2["topk_w"].view(torch.int32))
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("name,T", [("tiny", 64), ("q30", 96), ("dsv4", 300)])
def test_replay_of_other_ids_matches_the_oracle(name, T):
    inp = _inputs(name, T)
    if name == "dsv4":  # the oracle on 32 of the tokens
        from dataclasses import replace
        inp = replace(inp, cfg=replace(inp.cfg, T=32), x=inp.x[:32])
    cfg = inp.cfg
    T = cfg.T
    ref = oracle_forward(inp)
    # each token's K-th best expert replaced by its (K+1)-th (by the oracle's choice)
    order = np.argsort(-ref.choice, axis=1, kind="stable")
    ids = np.sort(np.concatenate([order[:, :cfg.K - 1], order[:, cfg.K:cfg.K + 1]], axis=1), axis=1).astype(np.int32)
    layer = make_layer(inp)
    x = to_dev(inp.x)
    od = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    out, tr = layer.forward(x, out_dtype=od, trace=True, replay_ids=to_dev(ids))
    torch.cuda.synchronize()
    rep = oracle_forward(inp, ids_override=ids)
    np.testing.assert_array_equal(to_host(tr["topk_ids"]), ids)
    np.testing.assert_allclose(to_host(tr["topk_w"]), rep.weights, rtol=2e-6, atol=1e-7)
    emu = oracle.combine_fp32(to_host(tr["y"]), to_host(tr["inv_pos"]), to_host(tr["topk_w"]),
                              to_host(tr["shared_out"]) if cfg.Is > 0 else None,
                              out="f32" if od == torch.float32 else "bf16")
    gout = to_host(out)
    assert np.array_equal(gout, emu)
    tol = 1e-5 if cfg.dtype == "f32" else 2e-2
    pr = check_layer_output(layer.with_tokens(T), tr, gout, rep.out, None, tol)
    _say(f"[replay] {name}-T{T} {json.dumps(pr)}")


def test_invalid_replayed_ids_are_masked():
    cfg = get_config("tiny")
    inp = make_inputs(cfg)
    ref = oracle_forward(inp)
    ids = ref.ids.copy()
    ids[3] = [-1, -1]          # a masked token of the recording
    ids[7] = [2, 2]            # repeated id
    ids[9] = [1, cfg.E]        # out of range
    layer = make_layer(inp)
    out, tr = layer.forward(to_dev(inp.x), out_dtype=torch.float32, trace=True, replay_ids=to_dev(ids))
    torch.cuda.synchronize()
    gi = to_host(tr["topk_ids"])
    o = to_host(out)
    for t in (3, 7, 9):
        assert np.all(gi[t] == -1) and np.all(o[t] == 0), t
    keep = np.setdiff1d(np.arange(cfg.T), [3, 7, 9])
    np.testing.assert_array_equal(gi[keep], ids[keep])
