"""Seeded draws for one MoE layer: hidden states, weights, bias, masks, shuffles.

All tensors are row-major.  bf16 values are returned as ``uint16`` bit
patterns, fp32 values as ``float32``.  Layouts:

  x            [T, D]
  w_router     [E, D]
  w_gate_up    [E, 2I, D]   rows 0..I-1 are the gate projection, I..2I-1 the up projection
  w_down       [E, D, I]
  w_gate_up_s  [2Is, D]     shared expert, same convention
  w_down_s     [D, Is]
  bias         [E] float32  selection bias (or None)
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

from .configs import (
    ROWS_PER_CHUNK,
    TID_BIAS,
    TID_PAD,
    TID_SHUFFLE,
    TID_W_DOWN,
    TID_W_DOWN_SHARED,
    TID_W_GATE_UP,
    TID_W_GATE_UP_SHARED,
    TID_W_ROUTER,
    TID_X,
    TID_ZIPF,
    TIE_TOKENS,
    LayerConfig,
)


def _rng(seed: int, tid: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, chunk])))


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16, nearest-even (inputs are finite)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = b + np.uint32(0x7FFF)
    r += (b >> np.uint32(16)) & np.uint32(1)
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(cfg: LayerConfig, a32: np.ndarray) -> np.ndarray:
    """Apply the config's value rounding, then its operand representation."""
    if cfg.value_dtype == "bf16":
        bits = _f32_to_bf16_bits(a32)
        return bits if cfg.dtype == "bf16" else bf16_bits_to_f32(bits)
    if cfg.dtype == "bf16":
        raise ValueError("a float32-valued layer cannot be run with bf16 operands")
    return np.ascontiguousarray(a32, dtype=np.float32)


def _normal(seed: int, tid: int, chunk: int, shape, std: float) -> np.ndarray:
    a = _rng(seed, tid, chunk).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _hidden_chunk(cfg: LayerConfig, c: int, tid: int, seed: int) -> np.ndarray:
    z = _normal(seed, tid, c, (ROWS_PER_CHUNK, cfg.D), 1.0 if cfg.x_dist == "rmsnorm" else cfg.x_std)
    if cfg.x_dist == "rmsnorm":
        # rows scaled to unit RMS, in float32, no epsilon and no gain
        rms = np.sqrt(np.mean(z * z, axis=1, dtype=np.float32), dtype=np.float32)
        z /= rms[:, None]
    return z


def hidden_states(cfg: LayerConfig, T: Optional[int] = None, threads: int = 0) -> np.ndarray:
    """x [T, D]; any prefix of the token pool is identical for every T."""
    T = cfg.T if T is None else T
    nchunks = (T + ROWS_PER_CHUNK - 1) // ROWS_PER_CHUNK
    out = np.empty((nchunks * ROWS_PER_CHUNK, cfg.D), dtype=np.float32)

    def fill(c):
        out[c * ROWS_PER_CHUNK:(c + 1) * ROWS_PER_CHUNK] = _hidden_chunk(cfg, c, TID_X, cfg.seed_x)

    _pmap(fill, range(nchunks), threads)
    x = out[:T]
    if cfg.zipf is not None:
        x[:, 0] = 1.0  # the channel that carries expert popularity
    if cfg.ties:
        _tie_rows(cfg, x)
    return _store(cfg, x)


def padding_rows(cfg: LayerConfig, n: int, stream: int = 0) -> np.ndarray:
    """n random rows drawn like the hidden states, for padding tests."""
    nchunks = max(1, (n + ROWS_PER_CHUNK - 1) // ROWS_PER_CHUNK)
    z = np.concatenate([_hidden_chunk(cfg, 1000 * stream + c, TID_PAD, cfg.seed_s) for c in range(nchunks)])[:n]
    if cfg.zipf is not None:
        z[:, 0] = 1.0
    return _store(cfg, z)


def shuffle_perm(cfg: LayerConfig, T: int, k: int) -> np.ndarray:
    """The k-th seeded permutation of T token positions (int64)."""
    return _rng(cfg.seed_s, TID_SHUFFLE, k).permutation(T)


# Tie construction for the tiny layer (8 experts, top-2).  Token 5 is the zero
# row, so all eight logits are exactly zero.  Tokens 17, 33 and 60 are one-hot
# rows (1.0 at column 0, 1, 2); their logits are then exactly the router
# column below, in any summation order.  The columns put a tie at ranks 2/3
# (the top-k boundary), at ranks 1/2 (inside the top-k) and a three-way tie at
# ranks 2/3/4.
_TIE_COLUMNS = {
    17: (0, [0.01, 0.03, 0.02, 0.02, -0.01, 0.0, -0.02, 0.005]),
    33: (1, [0.0, 0.04, -0.01, 0.04, 0.01, 0.02, -0.03, 0.0]),
    60: (2, [0.05, 0.01, 0.03, 0.0, 0.03, -0.02, 0.03, 0.01]),
}


def _tie_rows(cfg: LayerConfig, x: np.ndarray) -> None:
    if cfg.T <= 0:
        return
    for t in TIE_TOKENS:
        if t < x.shape[0]:
            x[t] = 0.0
    for t, (col, _) in _TIE_COLUMNS.items():
        if t < x.shape[0]:
            x[t, col] = 1.0


def router_weights(cfg: LayerConfig) -> np.ndarray:
    w = _normal(cfg.seed_w, TID_W_ROUTER, 0, (cfg.E, cfg.D), cfg.w_std)
    if cfg.zipf is not None:
        # expert e's softmax odds are multiplied by r_e^-zipf on every token,
        # r a seeded permutation of 1..E: Zipf-distributed expert popularity
        r = _rng(cfg.seed_w, TID_ZIPF, 0).permutation(cfg.E) + 1
        w[:, 0] = (-cfg.zipf * np.log(r.astype(np.float64))).astype(np.float32)
    if cfg.ties:
        assert cfg.E == 8, "the tie columns are written for 8 experts"
        for _, (col, vals) in _TIE_COLUMNS.items():
            w[:, col] = np.asarray(vals, dtype=np.float32)
    return _store(cfg, w)


def expert_weights(cfg: LayerConfig, e: int, shared: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """(gate_up [2I, D], down [D, I]) of routed expert e, or of the shared expert."""
    if shared:
        if cfg.Is == 0:
            raise ValueError("config has no shared expert")
        w1 = _normal(cfg.seed_w, TID_W_GATE_UP_SHARED, 0, (2 * cfg.Is, cfg.D), cfg.w_std)
        w2 = _normal(cfg.seed_w, TID_W_DOWN_SHARED, 0, (cfg.D, cfg.Is), cfg.w_std)
    else:
        w1 = _normal(cfg.seed_w, TID_W_GATE_UP, e, (2 * cfg.I, cfg.D), cfg.w_std)
        w2 = _normal(cfg.seed_w, TID_W_DOWN, e, (cfg.D, cfg.I), cfg.w_std)
    return _store(cfg, w1), _store(cfg, w2)


def selection_bias(cfg: LayerConfig) -> Optional[np.ndarray]:
    if cfg.bias is None:
        return None
    lo, hi = cfg.bias
    u = _rng(cfg.seed_b, TID_BIAS, 0).random(cfg.E, dtype=np.float32)
    return (np.float32(lo) + np.float32(hi - lo) * u).astype(np.float32)


def _pmap(fn, items, threads: int) -> None:
    items = list(items)
    n = threads or min(16, os.cpu_count() or 1)
    if n <= 1 or len(items) <= 1:
        for i in items:
            fn(i)
        return
    with ThreadPoolExecutor(n) as ex:
        for _ in ex.map(fn, items):
            pass


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: np.ndarray
    w_router: np.ndarray
    w_gate_up: np.ndarray
    w_down: np.ndarray
    w_gate_up_s: Optional[np.ndarray]
    w_down_s: Optional[np.ndarray]
    bias: Optional[np.ndarray]
    mask: Optional[np.ndarray] = None  # uint8 [T], 1 = kept token; None = all kept


def make_inputs(cfg: LayerConfig, T: Optional[int] = None, threads: int = 0) -> LayerInputs:
    """Every input of one layer forward (all experts' weights drawn)."""
    T = cfg.T if T is None else T
    x = hidden_states(cfg, T, threads)
    wdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    w1 = np.empty((cfg.E, 2 * cfg.I, cfg.D), dtype=wdt)
    w2 = np.empty((cfg.E, cfg.D, cfg.I), dtype=wdt)

    def fill(e):
        a, b = expert_weights(cfg, e)
        w1[e] = a
        w2[e] = b

    _pmap(fill, range(cfg.E), threads)
    w1s = w2s = None
    if cfg.Is > 0:
        w1s, w2s = expert_weights(cfg, 0, shared=True)
    return LayerInputs(cfg, x, router_weights(cfg), w1, w2, w1s, w2s, selection_bias(cfg))
