"""Backward of the layer against the CPU oracle, through the C ABI.

The RL-Kernel roadmap ("DSV4 Flash MoE Train-Inference Consistency Roadmap":
the scope list, forward + backward with a deterministic reduction order; the
issue-bucket table, a single-GPU forward + backward).  The oracle's backward
(float64, pinned to torch autograd) is fed the GPU's own picks, so the
comparison isolates the gradient arithmetic.

Acceptance.  The kernels feed three gradient operands to bf16 matrix
products: dY (the expert-output gradients), dH (the gate/up gradients) and dl
(the logits' gradient).  The oracle's grad_bf16 mode rounds at the same three
points, so against it only the float32 accumulation order and the rare
operand whose float32 and float64 values round to neighbouring bf16 values
(a flip) remain.  Normwise ||gpu - oracle|| <= TOL_NORM ||oracle||: flips are
sparse and the accumulation error is of order 2^-24 per term.  Elementwise
max |gpu - oracle| <= TOL_MAX times the oracle's RMS: a flip moves one
operand by one bf16 ulp (at most 2^-7 of it), and in a hot expert a single
product can be several times the gradient's RMS (one flip in dH of the
expert that holds every token of the softmax case is 3.3e-2 of the RMS, the
whole gap at that element to 1e-6).  Against the exact float64
gradient the three roundings (uniform over +-2^-9 relative, about 1.1e-3 rms
each, chained) give about 2e-3 normwise; the bound TOL_EXACT is four times
that.  Repeated calls must give the same bits, and a token's dx must not
depend on the other tokens of the batch (bitwise).
"""

import json
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from synth import get_config, make_inputs
from tests.gpu_util import make_layer, to_dev, to_host

pytestmark = pytest.mark.gpu

TOL_MAX = 5e-2
TOL_NORM = 2 ** -10
TOL_EXACT = 2 ** -7

CASES = [
    # config, reduced sizes, score override, masked
    ("dsv4", dict(T=256, D=512, E=16, K=4, I=256, Is=256), None, False),   # sigmoid + bias, renorm x2.5, shared
    ("dsv4", dict(T=160, D=512, E=16, K=4, I=256, Is=256), None, True),    # the same with masked tokens
    ("qnext", dict(T=200, D=256, E=64, K=8, I=128, Is=128), None, False),  # softmax, Zipf skew, shared
    ("q30", dict(T=130, D=256, E=16, K=4, I=192, Is=0), "sqrtsoftplus", False),  # N not a multiple of the tile
    ("dspark", dict(T=96, D=256, E=8, K=1, I=128, Is=0), None, False),     # top-1, no renorm, E = 8
    # 3000 rows: the router's and the shared expert's weight gradients are cut
    # into two K-slices (1536 + 1464 rows) summed in order
    ("dsv4", dict(T=3000, D=256, E=16, K=2, I=128, Is=128), None, False),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(name, dims, score, masked):
    cfg = replace(get_config(name), **dims)
    if score:
        cfg = replace(cfg, score=score)
    inp = make_inputs(cfg)
    if masked:
        rng = np.random.default_rng(5)
        inp.mask = (rng.random(cfg.T) > 0.3).astype(np.uint8)
    rng = np.random.default_rng(6)
    g32 = rng.standard_normal((cfg.T, cfg.D)).astype(np.float32)
    dout = (g32.view(np.uint32) + 0x7FFF + ((g32.view(np.uint32) >> 16) & 1)) >> 16
    return cfg, inp, dout.astype(np.uint16)


def _run(inp, dout):
    layer = make_layer(inp)
    x = to_dev(inp.x)
    mask = to_dev(inp.mask)
    _, tr = layer.forward(x, mask, trace=True)
    grads = layer.backward(x, to_dev(dout), tr, mask)
    torch.cuda.synchronize()
    return layer, tr, grads


@pytest.mark.parametrize("name,dims,score,masked", CASES)
def test_backward_against_oracle(name, dims, score, masked):
    cfg, inp, dout = _case(name, dims, score, masked)
    _say(f"[backward] {name} {dims} score={cfg.score} masked={masked}")
    layer, tr, grads = _run(inp, dout)
    ids = to_host(tr["topk_ids"])
    kw = dict(score=cfg.score, renorm=cfg.renorm, route_scale=cfg.route_scale, mask=inp.mask,
              shared_gate_up=inp.w_gate_up_s, shared_down=inp.w_down_s, bf16_mode=True)
    ref = oracle.backward(inp.x, inp.w_router, inp.w_gate_up, inp.w_down, dout, ids, grad_bf16=True, **kw)
    exact = oracle.backward(inp.x, inp.w_router, inp.w_gate_up, inp.w_down, dout, ids, **kw)
    rep = {}
    for k, v in grads.items():
        g = to_host(v).astype(np.float64)
        r, ex = ref[k], exact[k]
        rms = float(np.sqrt(np.mean(r * r)))
        rep[k] = (float(np.max(np.abs(g - r)) / rms), float(np.linalg.norm(g - r) / np.linalg.norm(r)),
                  float(np.linalg.norm(g - ex) / np.linalg.norm(ex)))
    _say(f"[backward] max/rms, norm, norm vs exact: {json.dumps(rep)}")
    for k, (emax, enorm, eexact) in rep.items():
        assert emax <= TOL_MAX and enorm <= TOL_NORM and eexact <= TOL_EXACT, (k, rep[k])
    if masked:
        assert np.all(to_host(grads["dx"])[inp.mask == 0] == 0)
    # experts no token picked get zero gradients
    counts = to_host(tr["counts"])
    for e in np.nonzero(counts == 0)[0]:
        assert np.all(to_host(grads["d_gate_up"][e]) == 0) and np.all(to_host(grads["d_down"][e]) == 0)
    # repeat: the same bits
    g2 = layer.backward(to_dev(inp.x), to_dev(dout), tr, to_dev(inp.mask))
    torch.cuda.synchronize()
    for k in grads:
        assert torch.equal(grads[k].view(torch.int32), g2[k].view(torch.int32)), k


def test_backward_dx_is_batch_invariant():
    """dx of a token is the same bits whether it is differentiated alone, in a
    prefix, or in the full batch (the weight gradients sum over the batch by
    definition and are only required to repeat)."""
    cfg, inp, dout = _case("dsv4", dict(T=256, D=512, E=16, K=4, I=256, Is=256), None, False)
    _, _, full = _run(inp, dout)
    dx_full = to_host(full["dx"])
    for T in (1, 37, 200):
        sub = replace(inp, cfg=replace(cfg, T=T), x=inp.x[:T])
        _, _, part = _run(sub, dout[:T])
        assert np.array_equal(to_host(part["dx"]).view(np.uint32), dx_full[:T].view(np.uint32)), T


def _grad_report(g, r, ex):
    g = np.asarray(g, dtype=np.float64)
    rms = float(np.sqrt(np.mean(r * r)))
    return (float(np.max(np.abs(g - r)) / rms), float(np.linalg.norm(g - r) / np.linalg.norm(r)),
            float(np.linalg.norm(g - ex) / np.linalg.norm(ex)))


@pytest.mark.parametrize("name", ["dsv4", "qnext"])
def test_backward_full_size_sampled(name):
    """A workload at full size — the DeepSeek-V4-Flash-like layer (T=32768,
    D=4096, 256 experts, top-6 sigmoid with selection bias, I=2048, one shared
    expert of 2048), as the benchmark times it, and the Qwen3-Next-like one
    (T=16384, D=2048, 512 experts, top-10 softmax with Zipf skew, I=512, shared
    512) — moe_backward over the whole batch.  dx of sampled tokens (a token's
    dx depends on that token alone) and the complete weight gradients of the
    most and the least loaded expert, against the oracle; the repeat is
    bitwise."""
    cfg = get_config(name)
    _say(f"[backward-full] drawing inputs T={cfg.T}")
    inp = make_inputs(cfg)
    rng = np.random.default_rng(7)
    g32 = rng.standard_normal((cfg.T, cfg.D), dtype=np.float32)
    u = g32.view(np.uint32)
    dout = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    del g32, u
    layer, tr, grads = _run(inp, dout)
    _say("[backward-full] forward + backward done")
    ids = to_host(tr["topk_ids"])
    counts = to_host(tr["counts"])
    kw = dict(score=cfg.score, renorm=cfg.renorm, route_scale=cfg.route_scale, bf16_mode=True)

    tok = np.sort(rng.choice(cfg.T, 8, replace=False))
    args = (inp.x[tok], inp.w_router, inp.w_gate_up, inp.w_down, dout[tok], ids[tok])
    sh = dict(shared_gate_up=inp.w_gate_up_s, shared_down=inp.w_down_s)
    ref = oracle.backward(*args, grad_bf16=True, **sh, **kw)["dx"]
    exact = oracle.backward(*args, **sh, **kw)["dx"]
    rep = {"dx_sampled": _grad_report(to_host(grads["dx"])[tok], ref, exact)}
    _say(f"[backward-full] dx of tokens {tok.tolist()}: {rep['dx_sampled']}")

    nz = np.nonzero(counts)[0]
    for e in (int(np.argmax(counts)), int(nz[np.argmin(counts[nz])])):
        ea = (e, inp.x, inp.w_router, inp.w_gate_up[e], inp.w_down[e], dout, ids)
        r1, r2 = oracle.backward_expert(*ea, grad_bf16=True, **kw)
        x1, x2 = oracle.backward_expert(*ea, **kw)
        rep[f"d_gate_up[{e}] rows={counts[e]}"] = _grad_report(to_host(grads["d_gate_up"][e]), r1, x1)
        rep[f"d_down[{e}] rows={counts[e]}"] = _grad_report(to_host(grads["d_down"][e]), r2, x2)
        _say(f"[backward-full] expert {e} ({counts[e]} rows) done")
    _say(f"[backward-full] max/rms, norm, norm vs exact: {json.dumps(rep)}")
    for k, (emax, enorm, eexact) in rep.items():
        assert emax <= TOL_MAX and enorm <= TOL_NORM and eexact <= TOL_EXACT, (k, rep[k])

    g2 = layer.backward(to_dev(inp.x), to_dev(dout), tr)
    torch.cuda.synchronize()
    for k in grads:
        assert torch.equal(grads[k].view(torch.int32), g2[k].view(torch.int32)), k


def test_backward_dx_shuffle_and_padding_invariant():
    """dx of a token is the same bits when the batch is shuffled and when it is
    padded with masked rows; the routed experts' weight gradients (each a sum
    over the expert's rows in token order, masked rows never among them) are
    the same bits under padding too."""
    cfg, inp, dout = _case("dsv4", dict(T=192, D=512, E=16, K=4, I=256, Is=256), None, False)
    _, _, base = _run(inp, dout)
    dx0 = to_host(base["dx"])
    # shuffle
    perm = np.random.default_rng(9).permutation(cfg.T)
    sh = replace(inp, x=inp.x[perm])
    _, _, g = _run(sh, dout[perm])
    assert np.array_equal(to_host(g["dx"]).view(np.uint32), dx0[perm].view(np.uint32))
    # padding: 64 extra rows (other hidden states, other output gradients), masked
    pad = 64
    rng = np.random.default_rng(10)
    xp = np.concatenate([inp.x, inp.x[rng.integers(0, cfg.T, pad)][:, ::-1].copy()])
    gp = np.concatenate([dout, dout[rng.integers(0, cfg.T, pad)]])
    mask = np.concatenate([np.ones(cfg.T, np.uint8), np.zeros(pad, np.uint8)])
    pd = replace(inp, cfg=replace(cfg, T=cfg.T + pad), x=xp, mask=mask)
    _, _, gpad = _run(pd, gp)
    dxp = to_host(gpad["dx"])
    assert np.array_equal(dxp[:cfg.T].view(np.uint32), dx0.view(np.uint32))
    assert np.all(dxp[cfg.T:] == 0)
    for k in ("d_gate_up", "d_down"):
        assert torch.equal(gpad[k].view(torch.int32), base[k].view(torch.int32)), k


def test_empty_batch():
    """T = 0: the forward succeeds and writes nothing; the backward's weight
    gradients are sums over no tokens, so zeros, written over whatever the
    buffers held (here NaN)."""
    import routing_grouped_gemm_gemv_amd.binding as B

    cfg, inp, _ = _case("dsv4", dict(T=8, D=256, E=16, K=4, I=128, Is=128), None, False)
    _say("[backward] empty batch")
    layer = make_layer(inp)
    x = torch.empty(0, cfg.D, dtype=torch.bfloat16, device="cuda")
    out, tr = layer.forward(x, trace=True)
    assert out.shape == (0, cfg.D)
    shape = layer.with_tokens(0)
    nan = float("nan")
    f32 = torch.float32
    grads = {
        "dx": torch.empty(0, cfg.D, dtype=f32, device="cuda"),
        "d_router": torch.full((cfg.E, cfg.D), nan, dtype=f32, device="cuda"),
        "d_gate_up": torch.full((cfg.E, 2 * cfg.I, cfg.D), nan, dtype=f32, device="cuda"),
        "d_down": torch.full((cfg.E, cfg.D, cfg.I), nan, dtype=f32, device="cuda"),
        "d_gate_up_shared": torch.full((2 * cfg.Is, cfg.D), nan, dtype=f32, device="cuda"),
        "d_down_shared": torch.full((cfg.D, cfg.Is), nan, dtype=f32, device="cuda"),
    }
    B.moe_backward(shape, layer.weights, x, None, tr, torch.empty(0, cfg.D, dtype=torch.bfloat16, device="cuda"),
                   grads, torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    for k, v in grads.items():
        assert torch.equal(v, torch.zeros_like(v)), k
