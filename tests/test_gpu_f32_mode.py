"""The fp32-operand mode on workload-shaped subsets, shared expert included.

The arXiv abstract ("From Expert Reduction to Behavioral Divergence",
Abstract) makes operand conversion and accumulator precision part of the
numerical contract, and the layer runs in two operand modes: bf16 operands
with fp32 accumulation, and fp32 operands.  Here the first 1024 tokens of the
DeepSeek-V4-Flash-like and Qwen3-Next-like layers run with fp32 operands (the
same bf16-valued inputs widened exactly) and are compared with the oracle in
float64 with no rounding anywhere:
  (a) ids bit-exact except near ties at the K boundary, weights to 2e-6;
  (b) the combine bit-exact against the float32 fold of the GPU's own y;
  (c) the layer output within 1e-5 of its RMS; the routed expert outputs and
      the shared expert output are each reported against their own RMS.
"""

import functools
import json

import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs
from tests.gpu_util import check_layer_output, f32_layer, make_layer, parity_report, routing_check, to_dev, to_host

pytestmark = pytest.mark.gpu

NTOK = 1024
TOL = 1e-5


@functools.lru_cache(maxsize=1)
def _inputs(name):
    print(f"[f32-mode] drawing {name} inputs (T={NTOK})", flush=True)
    return make_inputs(get_config(name, T=NTOK))


@pytest.mark.parametrize("name", ["dsv4", "qnext"])
def test_fp32_operand_layer_subset(name):
    inp = _inputs(name)
    cfg = inp.cfg
    layer = f32_layer(make_layer(inp))
    x = to_dev(inp.x).float()
    out, tr = layer.forward(x, out_dtype=torch.float32, trace=True)
    torch.cuda.synchronize()
    print(f"[f32-mode] {name}: forward done", flush=True)
    g = {k: to_host(v) for k, v in tr.items()}
    gout = to_host(out)
    ref = oracle.forward(inp.x, inp.w_router, inp.w_gate_up, inp.w_down, K=cfg.K, score=cfg.score,
                         renorm=cfg.renorm, route_scale=cfg.route_scale, bias=inp.bias,
                         shared_gate_up=inp.w_gate_up_s, shared_down=inp.w_down_s, bf16_mode=False)

    # (a)
    rc = routing_check(g["topk_ids"], ref)
    assert rc["mismatch_count"] == 0, rc
    same = np.all(g["topk_ids"] == ref.ids, axis=1)
    np.testing.assert_allclose(g["topk_w"][same], ref.weights[same], rtol=2e-6, atol=1e-7)
    pm = oracle.permute(g["topk_ids"], cfg.E)
    np.testing.assert_array_equal(g["inv_pos"], pm["inv_pos"])
    nv = int(pm["offsets"][-1])

    # (b)
    emu = oracle.combine_fp32(g["y"][:nv], g["inv_pos"], g["topk_w"], g["shared_out"], out="f32")
    assert np.array_equal(gout.view(np.uint32), emu.view(np.uint32))

    # (c) on tokens that routed as the oracle did (the others, exempt near ties,
    # against the oracle replaying the GPU's ids)
    ref_out, ref_y = ref.out.copy(), ref.y
    if not same.all():
        rep = oracle.forward(inp.x, inp.w_router, inp.w_gate_up, inp.w_down, K=cfg.K, score=cfg.score,
                             renorm=cfg.renorm, route_scale=cfg.route_scale, bias=inp.bias,
                             shared_gate_up=inp.w_gate_up_s, shared_down=inp.w_down_s, bf16_mode=False,
                             ids_override=g["topk_ids"])
        ref_out[~same] = rep.out[~same]
        ref_y = rep.y
    rows = parity_report(g["y"][:nv], ref_y)
    shared = parity_report(g["shared_out"], ref.shared)
    info = {k: rc[k] for k in ("exempt_count", "exempt_differing", "mismatch_count")}
    info.update({"routed_y_max_rel_rms": rows["max_rel_rms"], "shared_max_rel_rms": shared["max_rel_rms"]})
    pr = check_layer_output(layer.with_tokens(NTOK), tr, gout, ref_out, None, TOL, info)
    print(f"[f32-mode] {name}-T{NTOK} {json.dumps(pr)}", flush=True)
