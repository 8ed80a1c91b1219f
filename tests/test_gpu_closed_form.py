"""GPU parity against closed forms that do not go through the oracle.

Three special cases of the layer have results fixed by the mathematics alone,
computed here in float64 from the inputs:

* the token at global position 0 attends only to itself, so its attention
  output is its own value vector (rank 0, local row 0);
* with W_Q = 0 every score is 0 and the softmax is uniform over the visible
  keys, so the attention output at position p is the causal prefix mean of V
  over positions 0..p;
* with W1 = 0 the gate silu(n2 W1) is exactly 0, so the MLP adds exactly 0
  and the layer's output equals its attention half bit for bit.

Each runs over the attention paths: the pipelined bf16 kernel reading the
other ranks' K/V in place (C % 64 == 0), the copied-K/V path (ragged C),
query tiles split over key segments, other head dims, grouped K/V with the
rotary embedding, and fp32.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle.tsp_oracle as O
import synth
from gpu_harness import RankRun, f64, fill_kv, layer_dev, new_kv, say, to_dev
from parity import compare

pytestmark = pytest.mark.gpu


def _cfg(**kw):
    base = dict(name="closed", hidden=512, n_heads=4, head_dim=128, ffn=688, seq=2048, fold=4,
                ranks=(0,), layers=1, dtype="bf16", x_std=0.02)
    base.update(kw)
    return synth.LayerConfig(**base)


CASES = {
    "bf16_d128_inplace": _cfg(),                                      # C = 256
    "bf16_d128_ragged": _cfg(seq=1600),                               # C = 200
    "bf16_d128_split": _cfg(ffn=1024, seq=8192, fold=2),              # split key segments
    "bf16_d64_gqa2_rope": _cfg(hidden=256, head_dim=64, ffn=512, seq=1024, fold=2, n_kv_heads=2,
                               rope_theta=10000.0),
    "f32_d64": _cfg(hidden=128, n_heads=2, head_dim=64, ffn=344, seq=512, fold=2, dtype="f32"),
    "f32_d16_fold4": _cfg(hidden=64, n_heads=4, head_dim=16, ffn=172, seq=256, fold=4, dtype="f32"),
}


def _run(cfg, w):
    L = layer_dev(cfg, w)
    x_full = synth.gen_x_rows(cfg, 0, cfg.seq)
    pos = [O.zigzag_positions(cfg.seq, cfg.fold, r) for r in range(cfg.fold)]
    xs = [to_dev(x_full[p], cfg) for p in pos]
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    return L, x_full, pos, xs, kv


def _norm1(cfg, w, x):
    """RMSNorm-1 of rows x, as the kernels store it (the dtype's rounding)."""
    x = np.asarray(x, np.float64)
    n = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + cfg.eps) * np.asarray(w.g1, np.float64)
    return n


def _values(cfg, w, n):
    """V of every K/V head, [rows, Hkv*d], and the K/V head of each query head."""
    grp = cfg.n_heads // cfg.kv_heads
    return n @ np.asarray(w.wv, np.float64), [t // grp for t in range(cfg.n_heads)]


@pytest.mark.parametrize("case", sorted(CASES))
def test_first_position_attends_only_to_itself(case):
    cfg = CASES[case]
    say(f"[gpu] position 0 sees only itself ({case})")
    w = synth.gen_weights(cfg)
    L, x_full, pos, xs, kv = _run(cfg, w)
    x1 = RankRun(cfg, 0).attn(xs[0], L, kv)
    torch.cuda.synchronize()
    assert pos[0][0] == 0
    d = cfg.head_dim
    x0 = np.asarray(x_full[0:1], np.float64)
    v, kvh = _values(cfg, w, _norm1(cfg, w, x0))
    a = np.concatenate([v[:, kvh[t] * d:(kvh[t] + 1) * d] for t in range(cfg.n_heads)], axis=1)
    want = x0 + a @ np.asarray(w.wo, np.float64)
    ok, msg, _ = compare(cfg, f64(x1)[0:1], want, x0, x0)
    say(f"    x1 at position 0 against x + V(0) W_O: {msg}")
    assert ok, msg


@pytest.mark.parametrize("case", sorted(CASES))
def test_zero_queries_give_causal_prefix_mean(case):
    cfg = CASES[case]
    say(f"[gpu] W_Q = 0: attention is the causal prefix mean of V ({case})")
    w = synth.gen_weights(cfg)
    w = dataclasses.replace(w, wq=np.zeros_like(w.wq))
    L, x_full, pos, xs, kv = _run(cfg, w)
    d = cfg.head_dim
    x = np.asarray(x_full, np.float64)
    v, kvh = _values(cfg, w, _norm1(cfg, w, x))
    mean = np.cumsum(v, axis=0) / np.arange(1, cfg.seq + 1)[:, None]
    a = np.concatenate([mean[:, kvh[t] * d:(kvh[t] + 1) * d] for t in range(cfg.n_heads)], axis=1)
    want_all = x + a @ np.asarray(w.wo, np.float64)
    for r in range(cfg.fold):
        x1 = RankRun(cfg, r).attn(xs[r], L, kv)
        torch.cuda.synchronize()
        xr = x[pos[r]]
        ok, msg, _ = compare(cfg, f64(x1), want_all[pos[r]], xr, xr)
        say(f"    rank {r} x1 against x + prefix_mean(V) W_O: {msg}")
        assert ok, msg


@pytest.mark.parametrize("case", sorted(CASES))
def test_zero_gate_makes_the_mlp_exactly_zero(case):
    cfg = CASES[case]
    say(f"[gpu] W1 = 0: out == x1 bit for bit ({case})")
    w = synth.gen_weights(cfg)
    w = dataclasses.replace(w, w1=np.zeros_like(w.w1))
    L, x_full, pos, xs, kv = _run(cfg, w)
    for r in range(cfg.fold):
        run = RankRun(cfg, r)
        x1 = run.attn(xs[r], L, kv)
        out = run.layer(xs[r], L, kv)
        mlp = run.mlp(x1, L)
        torch.cuda.synchronize()
        assert torch.equal(out, x1), f"rank {r}: the zero gate changed the residual stream"
        assert torch.equal(mlp, x1), f"rank {r}: the MLP half alone is not the identity"
    say(f"    {cfg.fold} ranks bitwise equal")
