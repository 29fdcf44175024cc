"""The layer and its backward captured in HIP graphs: every replay, with eager
work and synchronisations between replays, gives the eager result bit for bit
(the library allocates nothing, issues no memsets and keeps no state, so a
captured launch sequence is the whole computation)."""

from dataclasses import replace

import numpy as np
import pytest
import torch

from synth import get_config, make_inputs
from tests.gpu_util import make_layer, to_dev

pytestmark = pytest.mark.gpu


def _inputs(name, **dims):
    cfg = replace(get_config(name), **dims)
    inp = make_inputs(cfg)
    return cfg, inp, make_layer(inp), to_dev(inp.x)


@pytest.mark.parametrize("name,dims", [("dsv4", dict(T=1024, D=512, E=32, K=6, I=256, Is=256)),
                                       ("qnext", dict(T=777))])
def test_forward_graph_replays(name, dims):
    cfg, inp, layer, x = _inputs(name, **dims)
    out = torch.empty(cfg.T, cfg.D, dtype=torch.bfloat16, device="cuda")
    layer.forward(x, out=out)  # allocates the workspace outside the capture
    torch.cuda.synchronize()
    ref = out.clone()
    got = torch.empty_like(out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, out=got)
    for i in range(3):
        got.fill_(7.0)
        layer.forward(x, out=out)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), i


def test_backward_graph_replays():
    from routing_grouped_gemm_gemv_amd import binding as B
    cfg, inp, layer, x = _inputs("dsv4", T=3000, D=256, E=16, K=2, I=128, Is=128)
    _, tr = layer.forward(x, trace=True)
    rng = np.random.default_rng(12)
    dout = torch.from_numpy(rng.standard_normal((cfg.T, cfg.D)).astype(np.float32)).to("cuda").to(torch.bfloat16)
    ref = layer.backward(x, dout, tr)
    torch.cuda.synchronize()
    shape = layer.with_tokens(cfg.T)
    grads = {k: torch.empty_like(v) for k, v in ref.items()}
    ws = torch.empty(B.backward_workspace_size(shape), dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.moe_backward(shape, layer.weights, x, None, tr, dout, grads, ws)
    for i in range(3):
        for v in grads.values():
            v.fill_(7.0)
        layer.backward(x, dout, tr)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(grads[k].view(torch.int32), ref[k].view(torch.int32)), (i, k)
