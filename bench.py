"""Benchmark of the sparse-MoE layer forward on one MI355X.

One step = one full layer forward (route, permute, routed experts, shared
expert, combine) over one batch of synthetic tokens already resident in HBM.
Prints one JSON line.  Default workload: the DeepSeek-V4-Flash-like layer
(T=32768, D=4096, 256 experts, top-6 sigmoid with selection bias and
route_scale 2.5, expert intermediate 2048, one shared expert of 2048), bf16
operands with fp32 accumulation.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s @1 GPU; expert-GEMM % bf16 MFMA peak; batch-invariant"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="dsv4", choices=["dsv4", "qnext", "q30", "dspark", "tiny"])
    ap.add_argument("--tokens", type=int, default=0, help="override T (0: the config's T)")
    ap.add_argument("--score", default=None, choices=["softmax", "sigmoid", "sqrtsoftplus"],
                    help="override the config's router score function")
    ap.add_argument("--groups", type=int, default=0, help="group-limited select: expert groups (0: the config's)")
    ap.add_argument("--topk-group", type=int, default=0, help="groups kept per token (with --groups)")
    ap.add_argument("--cpu-sample", type=int, default=4096, help="tokens timed on the CPU oracle (0: skip)")
    ap.add_argument("--no-invariance", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB buffer 5 times (reference kernel for the HBM byte counters)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of moe_forward captured in a HIP graph (launch overhead removed)")
    ap.add_argument("--ep-shard", type=int, default=0,
                    help="time moe_experts on the expert share of one of this many expert-parallel ranks")
    ap.add_argument("--backward", action="store_true",
                    help="time moe_backward (gradients of x and every weight) instead of the forward")
    ap.add_argument("--dense-reference", action="store_true",
                    help="only time the vendor dense bf16 GEMM (torch.mm) on the routed GEMMs' total shapes")
    return ap.parse_args()


COPY_BYTES = 1 << 30
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "dsv4_experts_traffic.json")
KERNEL_SOURCES = ("experts.hip", "common.hpp")


def kernel_source_hash() -> str:
    """sha256 of the sources of the grouped-GEMM kernels (host declarations excluded)."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "routing_grouped_gemm_gemv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM bytes per launch of the routed expert GEMMs from the committed counter
    record, or None when the kernels changed since the counters were taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("traffic_bytes_per_launch")


def copy_calibration():
    """A plain device copy of known size: FETCH_SIZE and WRITE_SIZE should each
    read COPY_BYTES per dispatch; the ratio scales the counters of other kernels."""
    import torch
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "dispatches": 5}), flush=True)


def dense_reference(cfg, rows: int, reps: int = 5):
    """Context, not the product: the library dense bf16 GEMM (hipBLASLt through
    torch.mm) on one matrix of all routed rows, for the gate_up shape
    [rows, D] x [D, 2I] and the down shape [rows, I] x [I, D], normal random
    operands.  The grouped kernels do the same FLOPs split over the experts."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    res = {}
    for name, (m, n, k) in (("gate_up", (rows, 2 * cfg.I, cfg.D)), ("down", (rows, cfg.D, cfg.I))):
        a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16, generator=g)
        b = (torch.randn(n, k, device="cuda", dtype=torch.bfloat16, generator=g) * 0.02).t()
        for _ in range(3):
            c = torch.mm(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c = torch.mm(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"shape_mnk": [m, n, k], "ms": ms, "tflops": 2.0 * m * n * k / ms / 1e9}
        del a, b, c
    total_ms = sum(r["ms"] for r in res.values())
    flops = sum(2.0 * r["shape_mnk"][0] * r["shape_mnk"][1] * r["shape_mnk"][2] for r in res.values())
    print(json.dumps({"dense_reference": res, "total_ms": total_ms, "tflops": flops / total_ms / 1e9}), flush=True)


def stage_bytes(cfg, T, nvalid_pairs):
    """Algorithmic HBM bytes of the route, permute and combine stages."""
    b = cfg.operand_bytes
    P = nvalid_pairs
    route = T * cfg.D * b + cfg.E * cfg.D * b + T * cfg.K * 8
    permute = T * cfg.K * 4 + 2 * P * 4 + (cfg.E * 2 + 1) * 4
    combine = P * cfg.D * b + (T * cfg.D * b if cfg.Is else 0) + T * cfg.D * 2 + T * cfg.K * 8
    return route, permute, combine


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.dense_reference:
        from synth import get_config
        cfg = get_config(args.config, T=args.tokens or None)
        dense_reference(cfg, cfg.T * cfg.K)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the layer is measured on exactly one GPU; --gpus must be 1 "
                                   "(the multi-GPU expert-parallel design is described, not built)"}))
        sys.exit(2)

    import numpy as np
    import torch

    import routing_grouped_gemm_gemv_amd as moe
    from synth import get_config, make_inputs

    cfg = get_config(args.config, T=args.tokens or None, score=args.score, n_group=args.groups or None,
                     topk_group=args.topk_group or None)
    T = cfg.T
    t0 = time.time()
    inp = make_inputs(cfg)
    log(f"inputs drawn in {time.time() - t0:.1f}s ({cfg.name}, T={T})")

    def dev(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(a).to("cuda")

    torch.cuda.set_device(0)
    shape = moe.Shape(T=T, D=cfg.D, E=cfg.E, K=cfg.K, I=cfg.I, Is=cfg.Is, score=cfg.score,
                      renorm=cfg.renorm, route_scale=cfg.route_scale, dtype=cfg.dtype,
                      n_group=cfg.n_group, topk_group=cfg.topk_group)
    x = dev(inp.x)
    layer = moe.MoeLayer(shape, dev(inp.w_router), dev(inp.w_gate_up), dev(inp.w_down),
                         dev(inp.w_gate_up_s), dev(inp.w_down_s), dev(inp.bias))
    out = torch.empty(T, cfg.D, dtype=torch.bfloat16, device="cuda")
    ws = layer.workspace(shape)
    torch.cuda.synchronize()
    log(f"uploaded; workspace {ws.numel() / 2**30:.2f} GiB")

    if args.backward:
        bench_backward(args, cfg, inp, layer, shape, x)
        return
    if args.ep_shard > 1:
        bench_ep_shard(args, cfg, layer, shape, x)
        return
    if args.graph:
        bench_graph(args, cfg, layer, x, out)
        return

    # ---- timed region 1: moe_forward, whole steps ---------------------------
    for _ in range(args.warmup):
        layer.forward(x, out=out)
    torch.cuda.synchronize()
    stream0 = torch.cuda.current_stream()
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_start = time.perf_counter()
    step_ev[0].record(stream0)
    for i in range(args.steps):
        layer.forward(x, out=out)
        step_ev[i + 1].record(stream0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall / args.steps * 1e3
    step_ms = [step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(args.steps)]

    # cold caches: a 1 GiB write between steps evicts the L2s and the 256 MB
    # last-level cache; each step timed alone with HIP events on its stream
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    cold_ms = []
    for _ in range(min(args.steps, 10)):
        flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream0)
        layer.forward(x, out=out)
        e1.record(stream0)
        torch.cuda.synchronize()
        cold_ms.append(e0.elapsed_time(e1))
    del flush
    log(f"moe_forward: {ms_per_step:.3f} ms/step")

    # ---- timed region 2: the same layer through the stage entry points, with
    # HIP events between stages on the stream the kernels run on -------------
    stream = torch.cuda.current_stream()
    tr = layer.new_trace(shape)
    B = moe.binding
    sh_shape = shape.replace(E=1, K=1, I=cfg.Is, Is=0, n_group=1, topk_group=1) if cfg.Is else None
    names = ["route", "permute", "experts_routed"] + (["experts_shared"] if cfg.Is else []) + ["combine"]

    def run_stages(evs):
        evs[0].record(stream)
        B.moe_route(shape, x, layer.weights["router"], layer.sel_bias, None, None, tr["topk_ids"], tr["topk_w"], ws)
        evs[1].record(stream)
        B.moe_permute(shape, tr["topk_ids"], tr["counts"], tr["offsets"], tr["perm_token"], tr["inv_pos"], ws)
        evs[2].record(stream)
        B.moe_experts(shape, x, tr["perm_token"], tr["offsets"], layer.weights["gate_up"], layer.weights["down"],
                      tr["y"], ws)
        evs[3].record(stream)
        i = 3
        shared = None
        if cfg.Is:
            B.moe_experts(sh_shape, x, None, None, layer.weights["gate_up_shared"], layer.weights["down_shared"],
                          tr["shared_out"], ws)
            i += 1
            evs[i].record(stream)
            shared = tr["shared_out"]
        B.moe_combine(shape, tr["y"], tr["inv_pos"], tr["topk_w"], shared, out)
        evs[i + 1].record(stream)

    for _ in range(max(1, args.warmup)):
        run_stages([torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)])
    torch.cuda.synchronize()
    all_evs = []
    for _ in range(args.steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        run_stages(evs)
        all_evs.append(evs)
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in all_evs])) for i, n in enumerate(names)}
    staged_total = float(np.mean([e[0].elapsed_time(e[-1]) for e in all_evs]))
    log("stages (ms): " + json.dumps({k: round(v, 4) for k, v in stage_ms.items()}))
    same_bits = bool(torch.equal(out.view(torch.int16), layer.forward(x).view(torch.int16)))

    counts = tr["counts"].cpu().numpy()
    P = int(counts.sum())
    gemm_flops = 6.0 * cfg.D * cfg.I * P
    shared_flops = 6.0 * cfg.D * cfg.Is * T
    layer_flops = 2.0 * cfg.D * cfg.E * T + gemm_flops + shared_flops
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    achieved = gemm_flops / (stage_ms["experts_routed"] * 1e-3) / 1e12
    rb, pb, cb = stage_bytes(cfg, T, P)
    hbm = {
        "route_gbs": rb / (stage_ms["route"] * 1e-3) / 1e9,
        "permute_gbs": pb / (stage_ms["permute"] * 1e-3) / 1e9,
        "combine_gbs": cb / (stage_ms["combine"] * 1e-3) / 1e9,
        "route_permute_combine_frac": (rb + pb + cb)
        / ((stage_ms["route"] + stage_ms["permute"] + stage_ms["combine"]) * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }

    # ---- batch invariance spot check: a prefix of the batch, bitwise --------
    invariant = None
    if not args.no_invariance and T > 1:
        Tp = max(1, min(T - 1, 1000))
        sub = layer.forward(x[:Tp].contiguous())
        full = layer.forward(x)
        invariant = bool(torch.equal(sub.view(torch.int16), full[:Tp].view(torch.int16)))
    torch.cuda.synchronize()

    # ---- CPU oracle on a bounded sample of the same workload ---------------
    # (timed, then compared with this run's GPU routing and output for the
    # same tokens: the parity fields of the line)
    cpu = None
    parity = None
    if args.cpu_sample > 0:
        n = min(args.cpu_sample, T)
        fwd = layer.forward(x[:n].contiguous(), trace=True)
        torch.cuda.synchronize()
        g_out, g_tr = fwd
        gpu = {"ids": g_tr["topk_ids"].cpu().numpy(), "w": g_tr["topk_w"].cpu().numpy(),
               "out": g_out.view(torch.int16).cpu().numpy().view(np.uint16)}
        cpu, parity = cpu_baseline(cfg, inp, n, gpu)

    line = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": float(np.median(step_ms)),
        "ms_per_step_min": float(np.min(step_ms)),
        "ms_per_step_cold_median": float(np.median(cold_ms)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; shapes and value distributions of the configs, random-init weights)",
        "config": {
            "workload": f"{cfg.name}-like MoE layer forward",
            "T": T, "D": cfg.D, "E": cfg.E, "K": cfg.K, "I": cfg.I, "Is": cfg.Is,
            "score": cfg.score, "renorm": cfg.renorm, "route_scale": cfg.route_scale,
            **({"n_group": cfg.n_group, "topk_group": cfg.topk_group} if cfg.n_group > 1 else {}),
            "selection_bias": cfg.bias is not None, "operands": cfg.dtype, "accumulate": "fp32",
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "moe_experts routed (grouped gate_up+SwiGLU GEMM, grouped down GEMM)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": recorded_traffic(f"{cfg.name}-T{T}") if cfg.name == "dsv4" else None,
        },
        "layer_tflops": layer_flops / (ms_per_step * 1e-3) / 1e12,
        "stage_ms": stage_ms,
        "staged_ms_per_step": staged_total,
        "stages_bitwise_equal_forward": same_bits,
        "hbm": hbm,
        "batch_invariant_prefix_check": invariant,
        "routed_pairs": P,
        "expert_load_max_over_mean": float(counts.max() / max(1e-9, counts.mean())),
        "expert_load": {"counts": [int(c) for c in counts], "min": int(counts.min()), "max": int(counts.max()),
                        "mean": float(counts.mean()), "empty_experts": int((counts == 0).sum())},
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_graph(args, cfg, layer, x, out):
    """moe_forward captured once in a HIP graph and replayed: the layer
    without host launch overhead (decode-sized batches are launch-bound).
    Every replay gives the eager bits (tests/test_gpu_graph.py)."""
    import numpy as np
    import torch

    layer.forward(x, out=out)  # the workspace exists before the capture
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, out=out)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_start = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        g.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    same = bool(torch.equal(out.view(torch.int16), ref.view(torch.int16)))
    ms = wall / args.steps * 1e3
    print(json.dumps({
        "metric": "MoE-layer tokens/s @1 GPU, moe_forward replayed from a HIP graph",
        "value": cfg.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": float(np.median(per)),
        "ms_per_step_min": float(np.min(per)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; shapes and value distributions of the configs, random-init weights)",
        "config": {"workload": f"{cfg.name}-like MoE layer forward, HIP graph replay", "T": cfg.T, "D": cfg.D,
                   "E": cfg.E, "K": cfg.K, "I": cfg.I, "Is": cfg.Is, "parallelism": "single GPU"},
        "replay_bitwise_equal_eager": same,
    }), flush=True)


def bench_ep_shard(args, cfg, layer, shape, x):
    """moe_experts on the experts one of P expert-parallel ranks would own
    (E/P experts, rank 0) with the rows the layer's routing sends them: the
    part of an expert-parallel layer one GPU runs, at its real shape.  Its
    rows are bitwise the full layer's (tests/test_gpu_ep_shard.py)."""
    import numpy as np
    import torch

    import routing_grouped_gemm_gemv_amd as moe
    B = moe.binding
    P = args.ep_shard
    if cfg.E % P:
        raise SystemExit(f"E = {cfg.E} does not split over {P} ranks")
    T = shape.T
    _, tr = layer.forward(x, trace=True)
    torch.cuda.synchronize()
    Es = cfg.E // P
    offs = tr["offsets"].cpu().numpy()
    rows = int(offs[Es])
    o_r = tr["offsets"][:Es + 1].contiguous()
    sh = shape.replace(E=Es, Is=0, n_group=1, topk_group=1)
    ws = layer.workspace(sh)
    y = torch.empty(T * cfg.K, cfg.D, dtype=torch.bfloat16, device="cuda")
    gu, dn = layer.weights["gate_up"][:Es], layer.weights["down"][:Es]

    def step():
        B.moe_experts(sh, x, tr["perm_token"], o_r, gu, dn, y, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_start = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = float(np.mean(per))
    same = bool(torch.equal(y[:rows].view(torch.int16), tr["y"][:rows].view(torch.int16)))
    flops = 6.0 * cfg.D * cfg.I * rows
    achieved = flops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": f"expert GEMMs of one of {P} expert-parallel ranks: TFLOP/s",
        "value": achieved,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "ms_per_step_median": float(np.median(per)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; the rows the layer's routing sends to rank 0's experts)",
        "config": {"workload": f"{cfg.name}-like layer, rank 0 of {P}: moe_experts", "T_total": T,
                   "experts": Es, "rows": rows, "D": cfg.D, "I": cfg.I, "parallelism": f"ep{P} (one rank)"},
        "roofline": {"kernel": "moe_experts (grouped gate_up+SwiGLU, grouped down)", "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None},
        "rows_bitwise_equal_full_layer": same,
    }), flush=True)


def bench_backward(args, cfg, inp, layer, shape, x):
    """One step = moe_backward over the trace of one forward: the gradients of
    the hidden states, the router and every expert weight (float32), from a
    seeded bf16 output gradient already resident in HBM."""
    import numpy as np
    import torch

    import routing_grouped_gemm_gemv_amd as moe
    B = moe.binding
    T = shape.T
    _, tr = layer.forward(x, trace=True)
    gen = torch.Generator(device="cuda").manual_seed(11)
    dout = torch.randn(T, cfg.D, device="cuda", generator=gen).to(torch.bfloat16)
    grads = layer.backward(x, dout, tr)  # allocates the gradients once
    ws = torch.empty(B.backward_workspace_size(shape), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"backward workspace {ws.numel() / 2**30:.2f} GiB, gradients "
        f"{sum(g.numel() for g in grads.values()) * 4 / 2**30:.2f} GiB")

    def step():
        B.moe_backward(shape, layer.weights, x, None, tr, dout, grads, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall / args.steps * 1e3
    ev_ms = e0.elapsed_time(e1) / args.steps
    log(f"moe_backward: {ms_per_step:.3f} ms/step (events {ev_ms:.3f})")
    first = {k: v.clone() for k, v in grads.items()}
    step()
    torch.cuda.synchronize()
    repeat_bitwise = all(torch.equal(first[k].view(torch.int32), grads[k].view(torch.int32)) for k in grads)

    P = int(tr["counts"].sum().item())
    # bf16 GEMM flops: H recomputed (2I x D), dA (I x D), dX (D x 2I), dW_down, dW_gate_up
    routed = 16.0 * cfg.D * cfg.I * P
    shared = 16.0 * cfg.D * cfg.Is * T
    router = 2.0 * 2.0 * cfg.D * cfg.E * T  # dx_r and dW_r (the float64 logits recompute not counted)
    flops = routed + shared + router
    achieved = flops / (ev_ms * 1e-3) / 1e12
    cpu = None
    n = min(args.cpu_sample, 16, T)
    if n > 0:
        import oracle
        ids = tr["topk_ids"][:n].cpu().numpy()
        g = dout[:n].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        oracle.backward(inp.x[:n], inp.w_router, inp.w_gate_up, inp.w_down, g, ids, score=cfg.score,
                        renorm=cfg.renorm, route_scale=cfg.route_scale, shared_gate_up=inp.w_gate_up_s,
                        shared_down=inp.w_down_s, bf16_mode=True)
        dt = time.perf_counter() - t0
        cpu = {"value": n / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"backward of the first {n} tokens of the same {cfg.name}-like layer, fp64 numpy "
                         f"oracle, {dt:.1f} s"}
    print(json.dumps({
        "metric": "MoE-layer backward tokens/s @1 GPU (dx, d_router, d_gate_up, d_down, shared)",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; random-init weights, seeded normal output gradient)",
        "config": {"workload": f"{cfg.name}-like MoE layer backward", "T": T, "D": cfg.D, "E": cfg.E,
                   "K": cfg.K, "I": cfg.I, "Is": cfg.Is, "score": cfg.score, "parallelism": "single GPU"},
        "roofline": {"kernel": "whole backward (bf16 MFMA GEMMs dominate)", "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None},
        "gemm_flops": flops,
        "repeat_bitwise": repeat_bitwise,
        "routed_pairs": P,
        "cpu_baseline": cpu,
    }), flush=True)


def cpu_baseline(cfg, inp, n, gpu):
    """The oracle, as it stands, on the first n tokens of the same layer.

    Returns the timing record and the parity of this run's GPU results for
    those tokens (gpu: their ids, weights and bf16 output bits from
    moe_forward on the same n tokens) against the oracle's: routing ids
    bit-exact except near ties (RL-Kernel roadmap, Problem 1: any mismatch
    reported), weights, and the layer output against the unrounded float64
    oracle in units of its RMS.
    """
    import numpy as np

    import oracle
    from threadpoolctl import threadpool_info

    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    cores = len(os.sched_getaffinity(0))
    log(f"cpu oracle on {n} tokens ({threads} BLAS threads, {cores} cores in affinity)")
    t0 = time.perf_counter()
    ref = oracle.forward(inp.x[:n], inp.w_router, inp.w_gate_up, inp.w_down, K=cfg.K, score=cfg.score,
                         renorm=cfg.renorm, route_scale=cfg.route_scale, bias=inp.bias,
                         shared_gate_up=inp.w_gate_up_s, shared_down=inp.w_down_s, bf16_mode=(cfg.dtype == "bf16"),
                         n_group=cfg.n_group, topk_group=cfg.topk_group)
    dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    timing = {
        "value": n / dt,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {n} tokens of the same {cfg.name}-like layer (all experts' weights), "
                  f"fp64 numpy oracle, {dt:.1f} s, {model}",
    }

    same = np.all(gpu["ids"] == ref.ids, axis=1)
    ok_w = np.abs(gpu["w"][same].astype(np.float64) - ref.weights[same]) <= 2e-6 * np.abs(ref.weights[same]) + 1e-7
    out32 = (gpu["out"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    cmp = same  # tokens routed alike: their outputs are comparable with the oracle's
    diff = np.abs(out32[cmp] - ref.out[cmp])
    rms = float(np.sqrt(np.mean(ref.out[cmp] ** 2))) if cmp.any() else 0.0
    rel = diff / rms if rms > 0 else diff
    # elements over 2e-2 RMS, and whether the final rounding accounts for
    # each: within one bf16 ulp of the float64 reference rounded once to bf16
    r64 = ref.out[cmp]
    r32 = r64.astype(np.float32)
    ru = r32.view(np.uint32)
    rne = (((ru + 0x7FFF + ((ru >> 16) & 1)) >> 16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    _, ex = np.frexp(rne)
    ulp = np.ldexp(1.0, np.where(rne == 0, -133, ex - 8))
    over = rel > 2e-2
    dist_ulp = np.abs(out32[cmp] - rne) / ulp
    parity = {
        "token_count": int(n),
        "mismatch_count": int((~same & ~ref.exempt).sum()),
        "exempt_count": int(ref.exempt.sum()),
        "exempt_differing": int((~same & ref.exempt).sum()),
        "weights_outside_rtol_2e-6": int((~ok_w).sum()),
        "output_compared_tokens": int(cmp.sum()),
        "output_rms": rms,
        "max_abs_diff": float(diff.max()) if diff.size else 0.0,
        "max_rel_rms": float(rel.max()) if rel.size else 0.0,
        "p99_rel_rms": float(np.percentile(rel, 99)) if rel.size else 0.0,
        "over_2e-2_rms_count": int(over.sum()),
        "over_2e-2_rms_max_ulp_from_rne_bf16_of_ref": float(dist_ulp[over].max()) if over.any() else 0.0,
        "share_within_1ulp_of_rne_bf16_of_ref": float(np.mean(dist_ulp <= 1.0)) if dist_ulp.size else 1.0,
        "reference": "oracle float64 layer output, unrounded; GPU value = the delivered bf16 output",
    }
    return timing, parity


if __name__ == "__main__":
    main()
