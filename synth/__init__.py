"""Seeded synthetic inputs for the sparse-MoE layer forward.

This package only draws numbers: hidden states, router and expert weights,
selection bias, padding masks and token shuffles, with the shapes and value
distributions of the workloads the pages describe.  It holds none of the
layer's arithmetic (no routing, no expert MLP, no combine), so that the CPU
oracle and the GPU path can both consume it without sharing any code with
each other.

Every tensor is drawn from numpy's PCG64 seeded by
``SeedSequence([seed, tensor_id, chunk])``; chunks are row blocks (or one
expert), so any prefix of tokens and any single expert can be regenerated
bit-for-bit on its own.  Draws are float32; bf16 tensors are the float32
draws rounded to nearest-even, stored as raw ``uint16`` bit patterns.
"""

from .configs import CONFIGS, LayerConfig, get_config
from .gen import (
    LayerInputs,
    bf16_bits_to_f32,
    expert_weights,
    hidden_states,
    make_inputs,
    padding_rows,
    shuffle_perm,
)

__all__ = [
    "CONFIGS",
    "LayerConfig",
    "get_config",
    "LayerInputs",
    "bf16_bits_to_f32",
    "expert_weights",
    "hidden_states",
    "make_inputs",
    "padding_rows",
    "shuffle_perm",
]
