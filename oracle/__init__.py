"""CPU oracle of the sparse-MoE layer forward -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, obviously-correct statement of what the GPU
path computes.  Only the test suite, the smoke check of ``__graft_entry__`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it.  The library and its
Python binding never call it, and it shares no code with them: the two meet
only in the seeded inputs of the ``synth`` package.

Precision: everything that is compared with a tolerance is computed in float64
(numpy matmul as the only library primitive).  The weighted combine, which the
pages make part of the numerical contract (operand conversion, accumulator
precision and reduction order), is emulated exactly in float32 with one IEEE
rounding per operation.

Pins (the tests that tie each function to something other than itself):
  router_logits      exact rational dot products on the tiny layer; one-hot/zero rows
  scores             torch.softmax / torch.sigmoid / softplus then sqrt (library
                     routines); sqrtsoftplus(0) = sqrt(log 2)
  select_topk        O(E^2) dominance count, exhaustive K-subsets, closed-form ties
  select_grouped     hand-derived examples (tests/golden); n_group = 1 and
                     topk_group = n_group reduce to select_topk; brute-force
                     group ranking with plain Python lists
  topk_weights       sum = route_scale, top-1 renorm = 1, zero row = 1/K
  route              the routing half of forward (logits .. weights) on its own;
                     equal to forward's routing fields (its pins are theirs)
  permute            numpy stable argsort; bijection and segment invariants
  expert_mlp         dense all-experts formulation with torch.nn.functional.silu;
                     E=1, K=1 reduces to a dense SwiGLU MLP
  round_bf16         exact rational round-half-even; torch's float32->bfloat16 cast
  combine_fp32       exact rational arithmetic rounded to float32 per operation;
                     720-order enumeration (360 classes) printed by the arXiv abstract
  combine_f64        exact rational sum rounded once (bf16 and float32); all 720
                     orders of six terms give one result
  backward           torch.autograd in float64 of an independently written
                     forward (straight-through bf16 rounding), every gradient;
                     masked tokens get none
No function is parity-unpinned.
"""

from .backward import backward, backward_expert
from .moe import (
    EXEMPT_REL_MARGIN,
    OracleResult,
    RouteResult,
    bf16_bits_of,
    combine_f64,
    combine_fp32,
    combine_orders,
    expert_mlp,
    forward,
    permute,
    round_bf16,
    route,
    router_logits,
    scores,
    select_grouped,
    select_topk,
    silu,
    topk_weights,
    widen,
)

__all__ = [
    "EXEMPT_REL_MARGIN",
    "backward",
    "backward_expert",
    "OracleResult",
    "RouteResult",
    "bf16_bits_of",
    "combine_f64",
    "combine_fp32",
    "combine_orders",
    "expert_mlp",
    "forward",
    "permute",
    "round_bf16",
    "route",
    "router_logits",
    "scores",
    "select_grouped",
    "select_topk",
    "silu",
    "topk_weights",
    "widen",
]
