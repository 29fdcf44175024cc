"""Layer shapes and input recipes of the synthetic workloads.

The shapes follow the models the pages discuss:
  * a tiny fp32 layer for exhaustive checks (8 experts, top-2) with four tokens
    whose router logits tie exactly, to exercise the lowest-id tie-break that
    the RL-Kernel roadmap ("DSV4 Flash MoE Train-Inference Consistency
    Roadmap", Problem 1: Routing Is A Discrete Decision) names as a risk;
  * the top-1 draft MoE of the SpecForge MoE-draft pull request (8 experts of
    intermediate 1536, top-1 without renormalisation, a selection bias);
  * a Qwen3-30B-A3B-like layer (the model of the UniRL parity pull request,
    "Supported case": BF16 compute, 256-token prompts);
  * a Qwen3-Next-like layer (the Qwen3.5-MoE family of the SpecForge pull
    request) with a shared expert and Zipf-skewed expert popularity;
  * a DeepSeek-V4-Flash-like layer (the model of the arXiv abstract "From
    Expert Reduction to Behavioral Divergence", six routed terms per token).
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

# tensor ids used in SeedSequence([seed, tensor_id, chunk])
TID_X = 0
TID_W_ROUTER = 1
TID_W_GATE_UP = 2
TID_W_DOWN = 3
TID_W_GATE_UP_SHARED = 4
TID_W_DOWN_SHARED = 5
TID_BIAS = 6
TID_PAD = 7
TID_SHUFFLE = 8
TID_ZIPF = 9

ROWS_PER_CHUNK = 1024  # hidden-state rows drawn per SeedSequence chunk


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int                      # tokens (the full pool for the Qwen3-30B-like sweep)
    D: int                      # hidden size
    E: int                      # routed experts
    K: int                      # experts per token
    I: int                      # routed expert SwiGLU intermediate
    Is: int                     # shared expert intermediate (0: no shared expert)
    dtype: str                  # operand mode: "bf16" (bf16 operands, fp32 accumulate) or "f32"
    value_dtype: str            # how draws are stored: "bf16" (rounded) or "f32"
    score: str                  # "softmax", "sigmoid" or "sqrtsoftplus"
    renorm: bool                # renormalise the selected weights to sum to 1
    route_scale: float          # multiplies the (renormalised) weights
    bias: Optional[Tuple[float, float]]  # selection bias U(lo, hi), or None
    x_dist: str                 # "normal" (N(0, x_std)) or "rmsnorm" (N(0,1) rows scaled to RMS 1)
    x_std: float
    w_std: float                # N(0, w_std) for every weight tensor
    zipf: Optional[float] = None  # Zipf exponent of expert popularity (router channel 0)
    ties: bool = False          # tiny only: tokens 5/17/33/60 get exact router ties
    seed_w: int = 0             # weights
    seed_x: int = 1             # hidden states
    seed_b: int = 2             # selection bias
    seed_s: int = 3             # shuffles and padding rows
    t_sweep: Tuple[int, ...] = field(default_factory=tuple)
    n_group: int = 1            # group-limited select: expert groups (1: none)
    topk_group: int = 1         # groups kept per token

    @property
    def P(self) -> int:
        return self.T * self.K

    def with_tokens(self, T: int) -> "LayerConfig":
        return replace(self, T=T)

    def flops_per_token(self) -> int:
        """Algorithmic FLOPs per valid token: router + routed SwiGLU + shared SwiGLU."""
        return 2 * self.D * self.E + 6 * self.D * self.I * self.K + 6 * self.D * self.Is

    @property
    def operand_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def has_shared(self) -> bool:
        return self.Is > 0


TIE_TOKENS = (5, 17, 33, 60)

CONFIGS = {
    "tiny": LayerConfig(
        name="tiny", T=64, D=128, E=8, K=2, I=256, Is=0, dtype="f32", value_dtype="f32",
        score="softmax", renorm=True, route_scale=1.0, bias=None,
        x_dist="normal", x_std=0.02, w_std=0.02, ties=True,
        seed_w=0, seed_x=0, seed_b=0, seed_s=0,
    ),
    "dspark": LayerConfig(
        name="dspark", T=4096, D=4096, E=8, K=1, I=1536, Is=0, dtype="bf16", value_dtype="bf16",
        score="softmax", renorm=False, route_scale=1.0, bias=(-0.05, 0.05),
        x_dist="normal", x_std=0.02, w_std=0.02,
    ),
    "q30": LayerConfig(
        name="q30", T=8192, D=2048, E=128, K=8, I=768, Is=0, dtype="bf16", value_dtype="bf16",
        score="softmax", renorm=True, route_scale=1.0, bias=None,
        x_dist="rmsnorm", x_std=1.0, w_std=0.02, t_sweep=(1, 256, 8192),
    ),
    "qnext": LayerConfig(
        name="qnext", T=16384, D=2048, E=512, K=10, I=512, Is=512, dtype="bf16", value_dtype="bf16",
        score="softmax", renorm=True, route_scale=1.0, bias=None,
        x_dist="rmsnorm", x_std=1.0, w_std=0.02, zipf=1.1,
    ),
    "dsv4": LayerConfig(
        name="dsv4", T=32768, D=4096, E=256, K=6, I=2048, Is=2048, dtype="bf16", value_dtype="bf16",
        score="sigmoid", renorm=True, route_scale=2.5, bias=(-0.05, 0.05),
        x_dist="rmsnorm", x_std=1.0, w_std=0.02,
    ),
}


def get_config(name: str, T: Optional[int] = None, dtype: Optional[str] = None, score: Optional[str] = None,
               n_group: Optional[int] = None, topk_group: Optional[int] = None) -> LayerConfig:
    """A named configuration; the optional arguments replace its token count,
    operand mode, score function or group-limited select."""
    cfg = CONFIGS[name]
    if score is not None:
        cfg = replace(cfg, score=score)
    if n_group is not None:
        cfg = replace(cfg, n_group=n_group, topk_group=topk_group if topk_group is not None else n_group)
    if T is not None:
        cfg = replace(cfg, T=T)
    if dtype is not None:
        # the operand mode changes; the drawn values keep the base config's rounding,
        # so an fp32-operand run of a bf16 layer sees the same bf16 values widened exactly
        cfg = replace(cfg, dtype=dtype)
    return cfg
