"""Batch invariance on the GPU: a token's ids, weights and output bits do not
depend on how many tokens share the batch, on padding, or on token order.

The RL-Kernel roadmap ("DSV4 Flash MoE Train-Inference Consistency Roadmap",
Problem 1 and the WS1 issue buckets) asks that routing metadata stay stable
across batch and padding sweeps and that any mismatch be reported; this is that
sweep on a Qwen3-30B-A3B-like layer (8192-token pool, 128 experts, top-8).
Self-consistency only: no oracle is needed.
"""

import numpy as np
import pytest
import torch

from synth import get_config, make_inputs, padding_rows, shuffle_perm
from tests.gpu_util import make_layer, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pool():
    cfg = get_config("q30")
    inp = make_inputs(cfg)
    layer = make_layer(inp)
    x = to_dev(inp.x)
    out, tr = layer.forward(x, trace=True)
    torch.cuda.synchronize()
    ref = {
        "out": to_host(out),
        "ids": to_host(tr["topk_ids"]),
        "w": to_host(tr["topk_w"]).view(np.uint32),
    }
    print(f"[invariance] pool T={cfg.T} ready", flush=True)
    return cfg, inp, layer, x, ref


def _run(layer, x, mask=None):
    out, tr = layer.forward(x, mask, trace=True)
    return to_host(out), to_host(tr["topk_ids"]), to_host(tr["topk_w"]).view(np.uint32)


def _same(T, got, ref, rows=None):
    o, i, w = got
    sel = slice(0, T) if rows is None else rows
    bad = np.nonzero(~(np.all(o[:T] == ref["out"][sel], axis=1) & np.all(i[:T] == ref["ids"][sel], axis=1)
                       & np.all(w[:T] == ref["w"][sel], axis=1)))[0]
    return bad


def test_every_batch_size_1_to_256(pool):
    cfg, inp, layer, x, ref = pool
    bad = {}
    for T in range(1, 257):
        b = _same(T, _run(layer, x[:T].contiguous()), ref)
        if b.size:
            bad[T] = b[:10].tolist()
    assert not bad, f"tokens whose bits changed with the batch size: {bad}"


@pytest.mark.parametrize("T", [257, 511, 1000, 2048, 4095, 4096, 8191])
def test_large_batch_sizes(pool, T):
    cfg, inp, layer, x, ref = pool
    b = _same(T, _run(layer, x[:T].contiguous()), ref)
    assert b.size == 0, b[:10]


@pytest.mark.parametrize("T", [1, 100, 1000, 4095])
@pytest.mark.parametrize("masked", [True, False])
def test_padding_to_multiple_of_128(pool, T, masked):
    cfg, inp, layer, x, ref = pool
    Tp = (T + 127) // 128 * 128 + 128
    pad = to_dev(padding_rows(cfg, Tp - T, stream=T))
    xp = torch.cat([x[:T], pad]).contiguous()
    mask = None
    if masked:
        m = torch.zeros(Tp, dtype=torch.uint8, device="cuda")
        m[:T] = 1
        mask = m
    o, i, w = _run(layer, xp, mask)
    b = _same(T, (o, i, w), ref)
    assert b.size == 0, b[:10]
    if masked:
        assert np.all(o[T:] == 0) and np.all(i[T:] == -1)


@pytest.mark.parametrize("k", [0, 1, 2])
def test_token_shuffles(pool, k):
    cfg, inp, layer, x, ref = pool
    perm = shuffle_perm(cfg, cfg.T, k)
    xs = x[torch.from_numpy(perm).to("cuda")].contiguous()
    o, i, w = _run(layer, xs)
    assert np.array_equal(o, ref["out"][perm])
    assert np.array_equal(i, ref["ids"][perm])
    assert np.array_equal(w, ref["w"][perm])


@pytest.mark.parametrize("name", ["dsv4", "qnext"])
def test_prefixes_across_the_decode_paths(name):
    """The small-batch paths (skinny experts, the shared expert's skinny path
    up to 64 rows, the small-batch router, the one-workgroup permute) give
    each token the same bits as the tiled paths: prefixes on both sides of
    every switch, against the 2048-token batch (DeepSeek-V4- and
    Qwen3-Next-like layers, both with a shared expert)."""
    cfg = get_config(name, T=2048)
    inp = make_inputs(cfg)
    layer = make_layer(inp)
    x = to_dev(inp.x)
    full, trf = layer.forward(x, trace=True)
    torch.cuda.synchronize()
    for T in (1, 2, 15, 16, 17, 63, 64, 65, 100, 200, 341, 342, 1000):
        sub, trs = layer.forward(x[:T].contiguous(), trace=True)
        torch.cuda.synchronize()
        assert torch.equal(sub.view(torch.int16), full[:T].view(torch.int16)), T
        assert torch.equal(trs["topk_ids"], trf["topk_ids"][:T]), T
        assert torch.equal(trs["topk_w"].view(torch.int32), trf["topk_w"][:T].view(torch.int32)), T


@pytest.mark.parametrize("name", ["q30", "qnext", "dsv4", "dspark"])
def test_router_tiles_give_the_same_bits(name):
    """The fused router picks its token tile from T and the CU count (larger
    tiles once every CU gets one).  A batch exactly at the switch runs the
    larger tile, the same batch without its last token the smaller one: the
    float32 logits, ids and weights of every common token are the same
    bits.  With at most 16 experts (the top-1 draft layer) the switch is
    between the small-batch router (up to 8192 tokens) and the fused one."""
    import routing_grouped_gemm_gemv_amd.binding as B
    from tests.gpu_util import make_layer

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    T = {"q30": 64 * cus, "qnext": 64 * cus, "dsv4": 128 * cus, "dspark": 8193}[name]
    cfg = get_config(name)
    inp = make_inputs(cfg, T=T)
    layer = make_layer(inp)
    x = to_dev(inp.x)
    print(f"[router tiles] {name} T={T} and {T - 1}", flush=True)
    res = []
    for n in (T, T - 1):
        shape = layer.with_tokens(n)
        ws = layer.workspace(shape)
        lg = torch.empty(n, cfg.E, dtype=torch.float32, device="cuda")
        ids = torch.empty(n, cfg.K, dtype=torch.int32, device="cuda")
        w = torch.empty(n, cfg.K, dtype=torch.float32, device="cuda")
        B.moe_route(shape, x[:n], layer.weights["router"], layer.sel_bias, None, lg, ids, w, ws)
        torch.cuda.synchronize()
        res.append((lg, ids, w))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a[: T - 1].view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("name", ["q30", "dsv4", "qnext"])
def test_single_token_down_and_combine_launch(name):
    """One token runs its experts' down projections and the combine in one
    launch; a batch of three runs them as separate launches.  The first token
    must give the same float32 output, the same expert outputs in the trace
    (y at its picks' rows, and the shared expert's row), and a masked single
    token a zero row with no picks."""
    cfg = get_config(name, T=3)
    inp = make_inputs(cfg)
    layer = make_layer(inp)
    x = to_dev(inp.x)
    o3, t3 = layer.forward(x, out_dtype=torch.float32, trace=True)
    o1, t1 = layer.forward(x[:1].contiguous(), out_dtype=torch.float32, trace=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(o1).view(np.uint32), to_host(o3)[:1].view(np.uint32))
    i1, i3 = to_host(t1["inv_pos"]), to_host(t3["inv_pos"])
    y1, y3 = to_host(t1["y"]), to_host(t3["y"])
    assert np.array_equal(to_host(t1["topk_ids"])[0], to_host(t3["topk_ids"])[0])
    for j in range(cfg.K):
        assert np.array_equal(y1[i1[0, j]], y3[i3[0, j]]), j
    if cfg.Is:
        assert np.array_equal(to_host(t1["shared_out"])[0], to_host(t3["shared_out"])[0])
    m = torch.zeros(1, dtype=torch.uint8, device="cuda")
    om, tm = layer.forward(x[:1].contiguous(), mask=m, trace=True)
    torch.cuda.synchronize()
    assert np.all(to_host(om) == 0) and np.all(to_host(tm["topk_ids"]) == -1)
    print(f"[decode-combine] {name}: T = 1 float32 output and trace equal to the 3-token batch's; masked row zero",
          flush=True)
