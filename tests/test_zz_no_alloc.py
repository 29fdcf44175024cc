"""moe_forward_noalloc (the allocation-free forward on the library's fixed
device scratch) against moe_forward with a caller workspace, bit for bit,
through the C ABI: two calls in a row, the second with a smaller batch, on
two layers; every boundary tensor of the trace and the output compared.
Shapes above the scratch size are refused before anything runs."""

import numpy as np
import pytest
import torch

from routing_grouped_gemm_gemv_amd import binding as B
from synth import get_config, make_inputs
from tests.gpu_util import make_layer, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    if t.dtype in (torch.float32, torch.int32):
        return t.view(torch.int32)
    return t.view(torch.int16)


def _run_pair(layer, x, T, out_dtype):
    shape = layer.with_tokens(T)
    xs = x[:T].contiguous()
    ref_out = torch.empty(T, shape.D, dtype=out_dtype, device="cuda")
    ref_tr = layer.new_trace(shape)
    B.moe_forward(shape, layer.weights, xs, layer.sel_bias, None, ref_out, layer.workspace(shape), ref_tr)
    out = torch.full((T, shape.D), 7.0, dtype=out_dtype, device="cuda")
    tr = {k: torch.full_like(v, -3) for k, v in layer.new_trace(shape).items()}
    B.moe_forward_noalloc(shape, layer.weights, xs, layer.sel_bias, None, out, tr)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref_out)), f"T={T}: output differs from moe_forward"
    nv = int(ref_tr["offsets"][-1])
    for k, v in ref_tr.items():
        a, b = (tr[k][:nv], v[:nv]) if k in ("perm_token", "y") else (tr[k], v)
        assert torch.equal(_bits(a), _bits(b)), f"T={T}: trace field {k} differs"
    # and without a trace: the boundary tensors then live in the scratch
    out2 = torch.full((T, shape.D), 5.0, dtype=out_dtype, device="cuda")
    B.moe_forward_noalloc(shape, layer.weights, xs, layer.sel_bias, None, out2)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out2), _bits(ref_out)), f"T={T}: output without trace differs"


@pytest.mark.parametrize("name,T1,T2", [("qnext", 384, 37), ("q30", 512, 1)])
def test_noalloc_forward_equals_forward_twice_shrinking(name, T1, T2):
    inp = make_inputs(get_config(name, T=T1))
    layer = make_layer(inp)
    x = to_dev(inp.x)
    _run_pair(layer, x, T1, torch.bfloat16)
    _run_pair(layer, x, T2, torch.bfloat16)
    print(f"[noalloc] {name}: T={T1} then T={T2} bitwise equal to moe_forward", flush=True)


def test_noalloc_refuses_shapes_above_the_scratch():
    inp = make_inputs(get_config("q30", T=64))
    layer = make_layer(inp)
    T = 8192
    shape = layer.with_tokens(T)
    assert B.workspace_size(shape) > B.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(T, shape.D, dtype=torch.bfloat16, device="cuda")
    out = torch.full((T, shape.D), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_noalloc(shape, layer.weights, x, None, None, out)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a refused call wrote its output"
