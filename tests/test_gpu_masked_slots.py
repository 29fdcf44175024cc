"""Partly masked rows through the public dispatch and combine entry points.

moe_permute accepts -1 in single slots of a token (and skips ids outside
[0, E) the same way); moe_combine must then skip those slots.  The dispatch
boundary of the RL-Kernel roadmap ("DSV4 Flash MoE Train-Inference
Consistency Roadmap", Problem 2: valid token counts and padding provenance)
and its reduction boundary (Problem 3) are checked here on ids the caller
makes, not the router's: the permutation against the oracle's counting sort,
the combine bit for bit against the oracle's float32 fold (and the float64
mode against the oracle's once-rounded sum), below and above the batch size
at which the combine switches kernels (16385 tokens), and the common tokens
of the two batches bitwise equal.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

E, K, D = 64, 6, 512
T_BIG = 16449    # above the combine kernel switch (16385 tokens); odd, so the
                 # two-token workgroups of the large-batch kernel end on a lone token
T_SMALL = 100    # below it; the first T_SMALL tokens of the big batch


def _ids(T):
    """K distinct ascending ids per token, then holes: single -1 slots, ids
    out of range (>= E or < -1), and a few tokens with every slot empty."""
    rng = np.random.default_rng(7)
    ids = np.sort(np.stack([rng.choice(E, K, replace=False) for _ in range(T)]), axis=1).astype(np.int32)
    hole = rng.random((T, K)) < 0.15
    bad = rng.random((T, K)) < 0.04
    ids[hole] = -1
    ids[bad & ~hole] = rng.choice(np.array([E, E + 3, 1 << 20, -2, -77], np.int32), int((bad & ~hole).sum()))
    for t in (3, 50, 1500, 16400):
        if t < T:
            ids[t] = -1
    return ids


def _per_slot_values(T):
    """bf16 expert-output values and float32 weights per (token, slot), so the
    same token sees the same terms whatever the batch and its rows."""
    rng = np.random.default_rng(11)
    vals = rng.standard_normal((T, K, D), dtype=np.float32)
    u = vals.view(np.uint32)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    w = rng.uniform(-2.0, 2.0, (T, K)).astype(np.float32)   # garbage weights in empty slots too
    shared = ((rng.standard_normal((T, D), dtype=np.float32).view(np.uint32) + 0x7FFF) >> 16).astype(np.uint16)
    return bits, w, shared


def _run(T, combine_mode, with_shared):
    from routing_grouped_gemm_gemv_amd import Shape
    from routing_grouped_gemm_gemv_amd import binding as B
    ids_all = _ids(T_BIG)
    vals_all, w_all, sh_all = _per_slot_values(T_BIG)
    ids, vals, w, sh = ids_all[:T], vals_all[:T], w_all[:T], sh_all[:T]
    shape = Shape(T=T, D=D, E=E, K=K, I=64, dtype="bf16", combine=combine_mode)
    ws = B.alloc_workspace(shape)
    d_ids = to_dev(ids)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.full((T * K,), -9, dtype=torch.int32, device="cuda")
    inv = torch.empty(T, K, dtype=torch.int32, device="cuda")
    B.moe_permute(shape, d_ids, counts, offsets, perm, inv, ws)
    torch.cuda.synchronize()

    # the dispatch: slots outside [0, E) are skipped like -1
    clean = np.where((ids >= 0) & (ids < E), ids, -1).astype(np.int32)
    pm = oracle.permute(clean, E)
    g_inv = to_host(inv)
    np.testing.assert_array_equal(to_host(counts), pm["counts"])
    np.testing.assert_array_equal(to_host(offsets), pm["offsets"])
    nv = int(pm["offsets"][-1])
    np.testing.assert_array_equal(to_host(perm)[:nv], pm["perm_token"])
    np.testing.assert_array_equal(g_inv, pm["inv_pos"])

    # expert outputs at the rows the dispatch gave each (token, slot)
    y = np.zeros((max(nv, 1), D), np.uint16)
    tt, jj = np.nonzero(g_inv >= 0)
    y[g_inv[tt, jj]] = vals[tt, jj]
    out32 = torch.empty(T, D, dtype=torch.float32, device="cuda")
    outbf = torch.empty(T, D, dtype=torch.bfloat16, device="cuda")
    d_y, d_w, d_sh = to_dev(y), to_dev(w), (to_dev(sh) if with_shared else None)
    B.moe_combine(shape, d_y, inv, d_w, d_sh, out32)
    B.moe_combine(shape, d_y, inv, d_w, d_sh, outbf)
    torch.cuda.synchronize()
    g32, gbf = to_host(out32), to_host(outbf)
    fn = oracle.combine_f64 if combine_mode == "f64" else oracle.combine_fp32
    ref_sh = sh if with_shared else None
    assert np.array_equal(g32.view(np.uint32), fn(y, g_inv, w, ref_sh, out="f32").view(np.uint32))
    assert np.array_equal(gbf, fn(y, g_inv, w, ref_sh, out="bf16"))
    assert np.all(g32[(g_inv < 0).all(axis=1)] == 0)
    return g32, gbf


@pytest.mark.parametrize("combine_mode", ["f32", "f64"])
@pytest.mark.parametrize("with_shared", [False, True])
def test_masked_slots_across_the_combine_switch(combine_mode, with_shared):
    s32, sbf = _run(T_SMALL, combine_mode, with_shared)
    b32, bbf = _run(T_BIG, combine_mode, with_shared)
    assert np.array_equal(s32.view(np.uint32), b32[:T_SMALL].view(np.uint32))
    assert np.array_equal(sbf, bbf[:T_SMALL])
    print(f"[masked-slots] combine={combine_mode} shared={with_shared}: T={T_SMALL} and T={T_BIG} "
          f"bit-exact against the oracle and equal on the common tokens", flush=True)


@pytest.mark.parametrize("k_slots,dim", [(1, 4608), (2, 256), (3, 1536), (8, 1536)])
def test_large_batch_combine_slot_counts(k_slots, dim):
    """The large-batch bf16 combine at slot counts and widths the layer
    workloads do not reach: K rounded up to 1, 2, 4 and 8 slots, and hidden
    sizes that end inside a thread's four-chunk round (256, 1536) or start a
    second round (4608); an odd batch, single empty slots and fully masked
    tokens; bit for bit against the oracle's float32 fold."""
    from routing_grouped_gemm_gemv_amd import Shape
    from routing_grouped_gemm_gemv_amd import binding as B
    T = 16391  # above the switch (16385 tokens), odd
    rng = np.random.default_rng(1000 + 10 * k_slots + dim)
    P = T * k_slots
    inv = rng.permutation(P).astype(np.int32).reshape(T, k_slots)
    inv[rng.random((T, k_slots)) < 0.05] = -1
    inv[::997] = -1
    vals = rng.standard_normal((P, dim), dtype=np.float32).view(np.uint32)
    y = ((vals + 0x7FFF + ((vals >> 16) & 1)) >> 16).astype(np.uint16)
    w = rng.uniform(-2.0, 2.0, (T, k_slots)).astype(np.float32)
    sv = rng.standard_normal((T, dim), dtype=np.float32).view(np.uint32)
    sh = ((sv + 0x7FFF + ((sv >> 16) & 1)) >> 16).astype(np.uint16)
    shape = Shape(T=T, D=dim, E=64, K=k_slots, I=64, dtype="bf16")
    d_y, d_inv, d_w, d_sh = to_dev(y), to_dev(inv), to_dev(w), to_dev(sh)
    out32 = torch.empty(T, dim, dtype=torch.float32, device="cuda")
    outbf = torch.empty(T, dim, dtype=torch.bfloat16, device="cuda")
    B.moe_combine(shape, d_y, d_inv, d_w, d_sh, out32)
    B.moe_combine(shape, d_y, d_inv, d_w, d_sh, outbf)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out32).view(np.uint32), oracle.combine_fp32(y, inv, w, sh, out="f32").view(np.uint32))
    assert np.array_equal(to_host(outbf), oracle.combine_fp32(y, inv, w, sh, out="bf16"))
    print(f"[combine-slots] K={k_slots} D={dim} T={T}: bit-exact against the oracle", flush=True)
