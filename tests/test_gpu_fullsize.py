"""Parity at the workloads' full sizes, in the launch configuration the benchmark
times (moe_forward over the whole batch, bf16 output), on sampled tokens the
oracle computes one by one; the permutation is checked in full."""

import json

import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs
from tests.gpu_util import make_layer, parity_report, routing_check, to_dev, to_host
from tests.oracle_bridge import oracle_forward

pytestmark = pytest.mark.gpu

SAMPLES = {"dsv4": 48, "qnext": 96, "q30": 128, "dspark": 128}


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

    # dispatch of the GPU's ids, all T*K pairs
    pm = oracle.permute(ids, cfg.E)
    np.testing.assert_array_equal(to_host(tr["counts"]), pm["counts"])
    np.testing.assert_array_equal(to_host(tr["offsets"]), pm["offsets"])
    nv = int(pm["offsets"][-1])
    np.testing.assert_array_equal(to_host(tr["perm_token"])[:nv], pm["perm_token"])
    np.testing.assert_array_equal(inv, pm["inv_pos"])

    # sampled tokens through the oracle
    rng = np.random.default_rng(1234)
    tok = np.sort(rng.choice(cfg.T, SAMPLES[name], replace=False))
    ref = oracle_forward(inp, tokens=tok)
    rc = routing_check(ids[tok], ref)
    assert rc["mismatch_count"] == 0, rc

    # combine on the GPU's own expert outputs for the sampled tokens
    y = to_host(tr["y"])
    rows = inv[tok]
    sub_y = y[rows.reshape(-1)]
    sub_inv = np.arange(rows.size, dtype=np.int32).reshape(rows.shape)
    sh = to_host(tr["shared_out"])[tok] if cfg.Is else None
    emu = oracle.combine_fp32(sub_y, sub_inv, w[tok], sh, out="bf16")
    gout = to_host(out)
    assert np.array_equal(gout[tok], emu)

    emu32 = oracle.combine_fp32(sub_y, sub_inv, w[tok], sh, out="f32")   # before the downcast
    ref_out = ref.out.copy()
    same = np.all(ids[tok] == ref.ids, axis=1)
    diff = np.nonzero(~same)[0]
    if diff.size:
        rep = oracle_forward(inp, tokens=tok, ids_override=ids[tok])
        ref_out[diff] = rep.out[diff]
    pr = parity_report(emu32, ref_out)
    g64 = oracle.widen(gout[tok])
    pr["bf16_out_max_rel_rms"] = float(np.max(np.abs(g64 - ref_out)) / pr["rms"])
    assert np.all(np.abs(g64 - ref_out) <= 2e-2 * pr["rms"] + 2.0 ** -8 * np.abs(ref_out)), pr
    counts = pm["counts"]
    pr.update({"exempt_count": rc["exempt_count"], "mismatch_count": rc["mismatch_count"],
               "load_max_over_mean": float(counts.max() / counts.mean()), "empty_experts": int((counts == 0).sum())})
    print(f"[fullsize] {name} {json.dumps(pr)}", flush=True)
    assert pr["max_rel_rms"] <= 2e-2, pr
