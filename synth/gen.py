"""Deterministic Gaussian inputs for a TSP layer.

Every tensor comes from its own numpy PCG64 stream seeded by
SeedSequence([seed, layer, tensor_id(, row_block)]).  Activations are drawn in
blocks of ROW_BLOCK rows so that any row range (for instance one rank's zigzag
chunks) can be produced without drawing the whole sequence.  Values are drawn
in float32 and, for bf16 workloads, rounded to the nearest bf16 (ties to even),
so the float32 arrays returned here hold exactly the bits both sides consume.

Weight layouts are the mathematical ones: Q = n @ wq with wq of shape
[h, h] (in, out); w1, w3 are [h, F]; w2 is [F, h].
"""
from dataclasses import dataclass
from typing import List

import numpy as np

ROW_BLOCK = 256

_TID = {"x": 0, "g1": 1, "g2": 2, "wq": 3, "wk": 4, "wv": 5, "wo": 6,
        "w1": 7, "w3": 8, "w2": 9}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are exact bfloat16 numbers."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _finish(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(a) if dtype == "bf16" else a.astype(np.float32)


def _rng(seed: int, layer: int, tid: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, tid, *extra])))


def gen_x_rows(cfg, lo: int, hi: int, layer: int = 0, seq_index: int = 0) -> np.ndarray:
    """Rows [lo, hi) of the input activations x_full [S, h] (float32) of
    sequence seq_index of a micro-batch (sequence 0 is the single-sequence
    stream; each other sequence draws from a stream of its own)."""
    extra = (seq_index,) if seq_index else ()
    if hi <= lo:
        return np.zeros((0, cfg.hidden), np.float32)
    out = np.empty((hi - lo, cfg.hidden), np.float32)
    b0, b1 = lo // ROW_BLOCK, (hi - 1) // ROW_BLOCK
    for b in range(b0, b1 + 1):
        rows = min(ROW_BLOCK, cfg.seq - b * ROW_BLOCK)
        blk = _rng(cfg.seed, layer, _TID["x"], b, *extra).standard_normal((rows, cfg.hidden),
                                                                          np.float32)
        blk *= np.float32(cfg.x_std)
        s, e = max(lo, b * ROW_BLOCK), min(hi, b * ROW_BLOCK + rows)
        out[s - lo:e - lo] = blk[s - b * ROW_BLOCK:e - b * ROW_BLOCK]
    return _finish(out, cfg.dtype)


def gen_rows(cfg, positions: np.ndarray, layer: int = 0, seq_index: int = 0) -> np.ndarray:
    """x_full rows at arbitrary global positions (in the order given)."""
    positions = np.asarray(positions, dtype=np.int64)
    if positions.size == 0:
        return np.zeros((0, cfg.hidden), np.float32)
    lo, hi = int(positions.min()), int(positions.max()) + 1
    # Draw the covering blocks once, then gather.
    blk = gen_x_rows(cfg, lo, hi, layer, seq_index)
    return blk[positions - lo]


def gen_gamma(cfg, which: str, layer: int = 0) -> np.ndarray:
    h = cfg.hidden
    if cfg.gamma == "ones":
        g = np.ones(h, np.float32)
    else:
        g = 1.0 + 0.1 * _rng(cfg.seed, layer, _TID[which]).standard_normal(h, np.float32)
    return _finish(g, cfg.dtype)


@dataclass
class LayerWeights:
    g1: np.ndarray  # [h]
    wq: np.ndarray  # [h, h]
    wk: np.ndarray  # [h, Hkv*d]
    wv: np.ndarray  # [h, Hkv*d]
    wo: np.ndarray  # [h, h]
    g2: np.ndarray  # [h]
    w1: np.ndarray  # [h, F]  gate branch (passed through silu)
    w3: np.ndarray  # [h, F]  linear branch
    w2: np.ndarray  # [F, h]  down projection


def gen_weights(cfg, layer: int = 0) -> LayerWeights:
    h, F = cfg.hidden, cfg.ffn
    hk = (cfg.n_kv_heads or cfg.n_heads) * cfg.head_dim
    std = np.float32(cfg.w_std)

    def w(name, shape):
        return _finish(_rng(cfg.seed, layer, _TID[name]).standard_normal(shape, np.float32) * std,
                       cfg.dtype)

    return LayerWeights(
        g1=gen_gamma(cfg, "g1", layer), wq=w("wq", (h, h)), wk=w("wk", (h, hk)),
        wv=w("wv", (h, hk)), wo=w("wo", (h, h)), g2=gen_gamma(cfg, "g2", layer),
        w1=w("w1", (h, F)), w3=w("w3", (h, F)), w2=w("w2", (F, h)))


def gen_stack(cfg) -> List[LayerWeights]:
    return [gen_weights(cfg, l) for l in range(cfg.layers)]
