"""Expert parallelism as one GPU can show it: each rank's share of the experts
run on its own through moe_experts gives, bit for bit, the expert-output rows
the whole layer computes (the RL-Kernel roadmap's EP consistency asks that
the dispatch layout not change results; every expert row comes from a
row-independent kernel with a fixed k order, so the share a rank holds
cannot change its rows)."""

import pytest
import torch

from synth import get_config, make_inputs
from tests.gpu_util import make_layer, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T,ranks", [("dsv4", 4096, 8), ("qnext", 2048, 4), ("q30", 1000, 8)])
def test_expert_shards_equal_the_layer(name, T, ranks):
    from routing_grouped_gemm_gemv_amd import binding as B
    cfg = get_config(name, T=T)
    print(f"[ep-shard] {name} T={T} ranks={ranks}", flush=True)
    inp = make_inputs(cfg)
    layer = make_layer(inp)
    x = to_dev(inp.x)
    _, tr = layer.forward(x, trace=True)
    torch.cuda.synchronize()
    offs = tr["offsets"].cpu()
    Es = cfg.E // ranks
    shape = layer.with_tokens(T).replace(E=Es, Is=0)
    ws = layer.workspace(shape)
    for r in range(ranks):
        lo, hi = int(offs[r * Es]), int(offs[(r + 1) * Es])
        o_r = (tr["offsets"][r * Es:(r + 1) * Es + 1] - lo).contiguous()
        y_r = torch.full((T * cfg.K, cfg.D), -7.0, dtype=torch.bfloat16, device="cuda")
        B.moe_experts(shape, x, tr["perm_token"][lo:], o_r, layer.weights["gate_up"][r * Es:(r + 1) * Es],
                      layer.weights["down"][r * Es:(r + 1) * Es], y_r, ws)
        torch.cuda.synchronize()
        assert torch.equal(y_r[:hi - lo].view(torch.int16), tr["y"][lo:hi].view(torch.int16)), r
    print(f"[ep-shard] {name}: {ranks} shards bitwise equal", flush=True)
