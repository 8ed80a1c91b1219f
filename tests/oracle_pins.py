"""Pins of the CPU oracle: checks against facts fixed outside the oracle.

Each pin takes the oracle module as its argument, so the same pins run both
against the real oracle (tests/test_oracle.py) and against copies of it with
a planted mistake (the mutation tests), where at least one pin must fail.

What the pins rest on:
  * the tiny workload's zigzag statement (rank 1 of 4 holds chunks 1 and 6),
    stored with its citation in tests/golden/zigzag_tiny_rank1.txt;
  * closed forms: the causal pair count per rank, the FLOP identity (same
    per-device compute as TP and SP, section 3 of the TSP page);
  * an independent library: torch's rms_norm, silu and causal
    scaled_dot_product_attention in float64, and a torch composition of the
    unsharded layer written separately from the oracle;
  * brute force: a pure-Python double loop for attention, and the literal
    D-rank schedule (broadcast / all-gather / ring, section 2 of the TSP page)
    against the unsharded layer;
  * special cases: the first position sees only itself; zero queries give
    the causal prefix mean of V; a zero W1 turns the MLP off.
"""
import math
import os

import numpy as np
import torch
import torch.nn.functional as Fn

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TINY = synth.get_config("tiny_fp32")


def _rng(seed):
    return np.random.default_rng(seed)


def _weights(cfg, layer=0, gamma="normal"):
    return synth.gen_weights(cfg.with_(gamma=gamma), layer)


def _x(cfg, layer=0):
    return synth.gen_x_rows(cfg, 0, cfg.seq, layer)


# ---------------------------------------------------------------- zigzag

def pin_zigzag_statement(o):
    with open(os.path.join(GOLDEN, "zigzag_tiny_rank1.txt")) as f:
        lines = [l for l in f if l.strip() and not l.startswith("#")]
    S, D, r = map(int, lines[0].split())
    want = np.array([int(t) for l in lines[1:] for t in l.split()])
    got = o.zigzag_positions(S, D, r)
    assert np.array_equal(got, want), "zigzag holdings differ from the tiny workload statement"
    assert tuple(o.zigzag_chunks(D, r)) == (1, 6)


def pin_zigzag_partition(o):
    for S, D in [(16, 1), (16, 2), (64, 4), (256, 4), (96, 3), (1024, 8)]:
        allpos = np.concatenate([o.zigzag_positions(S, D, r) for r in range(D)])
        assert np.array_equal(np.sort(allpos), np.arange(S)), (S, D)
        for r in range(D):
            p = o.zigzag_positions(S, D, r)
            assert p.size == S // D
            assert np.all(np.diff(p) > 0), "local rows must be in ascending global order"


def pin_zigzag_balance(o):
    """Every rank does the same causal work: C^2 (2D-1) + C (C+1) pairs."""
    for S, D in [(16, 1), (64, 2), (256, 4), (16384, 8), (65536, 8), (131072, 8), (32768, 4)]:
        C = S // (2 * D)
        closed = C * C * (2 * D - 1) + C * (C + 1)
        pairs = [o.causal_pairs(S, D, r) for r in range(D)]
        assert all(p == closed for p in pairs), (S, D, pairs, closed)
        assert sum(pairs) == S * (S + 1) // 2
        # brute-force count at small sizes, from the visibility rule itself
        if S <= 256:
            for r in range(D):
                pos = o.zigzag_positions(S, D, r)
                brute = sum(1 for p in pos for k in range(S) if k <= p)
                assert brute == pairs[r]


def pin_unzigzag(o):
    S, D = 64, 4
    x = np.arange(S * 3, dtype=np.float64).reshape(S, 3)
    parts = [x[o.zigzag_positions(S, D, r)] for r in range(D)]
    assert np.array_equal(o.unzigzag(parts, S, D), x)


# ---------------------------------------------------------------- textbook pieces

def pin_rmsnorm_torch(o):
    rng = _rng(1)
    x = rng.standard_normal((37, 64))
    g = 1 + 0.1 * rng.standard_normal(64)
    want = Fn.rms_norm(torch.from_numpy(x), (64,), weight=torch.from_numpy(g), eps=1e-5).numpy()
    assert np.allclose(o.rmsnorm(x, g, 1e-5), want, rtol=1e-12, atol=1e-12)
    # a constant row c*1 normalises to sign(c) * |c| / sqrt(c^2 + eps)
    c = -0.3
    got = o.rmsnorm(np.full((1, 8), c), np.ones(8), 1e-5)
    assert np.allclose(got, c / math.sqrt(c * c + 1e-5), rtol=1e-14)


def pin_silu_torch(o):
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(o.silu(z), Fn.silu(torch.from_numpy(z)).numpy(), rtol=1e-13, atol=1e-300)


def pin_attention_torch(o):
    rng = _rng(2)
    for S, d in [(1, 16), (7, 16), (200, 32), (130, 128)]:
        q, k, v = (rng.standard_normal((S, d)) for _ in range(3))
        want = Fn.scaled_dot_product_attention(*(torch.from_numpy(t)[None] for t in (q, k, v)),
                                               is_causal=True)[0].numpy()
        got = o.causal_attention(q, np.arange(S), k, v, block=64)
        assert np.allclose(got, want, rtol=1e-11, atol=1e-12), (S, d)
        # a subset of queries (one rank's zigzag rows) sees the same keys
        if S >= 8 and S % 8 == 0:
            rows = o.zigzag_positions(S, 4, 1)
            got = o.causal_attention(q[rows], rows, k, v, block=5)
            assert np.allclose(got, want[rows], rtol=1e-11, atol=1e-12)


def pin_attention_loops(o):
    """Pure-Python double loop over positions with math.exp."""
    rng = _rng(3)
    S, d = 11, 4
    q, k, v = (rng.standard_normal((S, d)) for _ in range(3))
    want = np.zeros((S, d))
    for p in range(S):
        s = [sum(q[p, e] * k[j, e] for e in range(d)) / math.sqrt(d) for j in range(p + 1)]
        m = max(s)
        wts = [math.exp(t - m) for t in s]
        z = sum(wts)
        for e in range(d):
            want[p, e] = sum(wts[j] * v[j, e] for j in range(p + 1)) / z
    assert np.allclose(o.causal_attention(q, np.arange(S), k, v, block=4), want, rtol=1e-12, atol=1e-13)


def pin_attention_special(o):
    rng = _rng(4)
    S, d = 50, 16
    q, k, v = (rng.standard_normal((S, d)) for _ in range(3))
    got = o.causal_attention(q, np.arange(S), k, v)
    assert np.allclose(got[0], v[0], rtol=1e-13), "position 0 sees only itself"
    # zero queries -> uniform weights over the visible prefix -> prefix mean
    got = o.causal_attention(np.zeros_like(q), np.arange(S), k, v)
    pref = np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None]
    assert np.allclose(got, pref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- whole layer

def torch_layer(x, w, H, eps):
    """The unsharded pre-norm layer composed from torch library routines."""
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    X = T(x)
    S, h = X.shape
    d = h // H
    n1 = Fn.rms_norm(X, (h,), weight=T(w.g1), eps=eps)
    heads = lambda m: (n1 @ T(m)).reshape(S, H, d).transpose(0, 1).contiguous()
    a = Fn.scaled_dot_product_attention(heads(w.wq), heads(w.wk), heads(w.wv), is_causal=True)
    x1 = X + a.transpose(0, 1).reshape(S, h) @ T(w.wo)
    n2 = Fn.rms_norm(x1, (h,), weight=T(w.g2), eps=eps)
    return (x1 + (Fn.silu(n2 @ T(w.w1)) * (n2 @ T(w.w3))) @ T(w.w2)).numpy()


def pin_layer_torch(o):
    for cfg in [TINY, TINY.with_(seq=64, fold=2, hidden=32, n_heads=2, ffn=40)]:
        w, x = _weights(cfg), _x(cfg)
        want = torch_layer(x, w, cfg.n_heads, cfg.eps)
        got = o.layer_unsharded(x, w, cfg.n_heads, cfg.eps)
        assert o.rel_fro(got, want) < 1e-12, o.rel_fro(got, want)
        # restricted rows, the attention half and the MLP half agree too
        rows = o.zigzag_positions(cfg.seq, cfg.fold, 1)
        assert o.rel_fro(o.layer_rows(x, w, cfg.n_heads, cfg.eps, rows), want[rows]) < 1e-12
        x1 = o.attention_block_rows(x, w, cfg.n_heads, cfg.eps, np.arange(cfg.seq))
        assert o.rel_fro(o.mlp_block(x1, w, cfg.eps), want) < 1e-12
        assert o.rel_fro(o.rank_share(x, w, cfg.n_heads, cfg.eps, cfg.seq, cfg.fold, 1),
                         want[rows]) < 1e-12


def pin_mlp_zero_gate(o):
    cfg = TINY
    w = _weights(cfg)
    w.w1 = np.zeros_like(w.w1)
    x = _x(cfg)
    x1 = o.attention_block_rows(x, w, cfg.n_heads, cfg.eps, np.arange(cfg.seq))
    assert np.array_equal(o.layer_unsharded(x, w, cfg.n_heads, cfg.eps), x1)


def pin_fold_bruteforce(o):
    """The literal D-rank schedule, un-zigzagged, equals the unsharded layer."""
    cases = [TINY, TINY.with_(seq=16, fold=1), TINY.with_(seq=64, fold=2),
             TINY.with_(seq=16, fold=4, ffn=176), TINY.with_(seq=64, fold=4, n_heads=8, head_dim=8)]
    for cfg in cases:
        w, x = _weights(cfg), _x(cfg)
        want = o.layer_unsharded(x, w, cfg.n_heads, cfg.eps)
        parts = o.fold_schedule(x, w, cfg.n_heads, cfg.eps, cfg.fold)
        assert o.rel_fro(o.unzigzag(parts, cfg.seq, cfg.fold), want) < 1e-12, cfg


def pin_mlp_partials(o):
    """Partial MLP outputs of the D shards sum to the full MLP (no all-reduce)."""
    for cfg in [TINY, TINY.with_(ffn=176, fold=8), TINY.with_(fold=1)]:
        w = _weights(cfg)
        n = _rng(5).standard_normal((33, cfg.hidden))
        full = o.swiglu_mlp(n, w.w1, w.w3, w.w2)
        parts = o.mlp_partials(n, w, cfg.fold)
        assert len(parts) == cfg.fold
        assert o.rel_fro(sum(parts), full) < 1e-13


def pin_stack(o):
    cfg = TINY.with_(layers=2, seq=64, fold=2)
    ws = [_weights(cfg, l) for l in range(2)]
    x = _x(cfg)
    want = torch_layer(torch_layer(x, ws[0], cfg.n_heads, cfg.eps), ws[1], cfg.n_heads, cfg.eps)
    rows = np.array([0, 5, 17, 63])
    assert o.rel_fro(o.stack_rows(x, ws, cfg.n_heads, cfg.eps, rows), want[rows]) < 1e-12


def pin_flops(o):
    """Sum of the ranks' FLOPs equals the unsharded layer's (equal per-device
    compute), and each rank's share is exactly 1/D of it."""
    for h, F, S, D in [(64, 172, 256, 4), (4096, 11008, 65536, 8), (4096, 11008, 32768, 4)]:
        per = [o.flops_rank(h, F, S, D, r) for r in range(D)]
        assert sum(per) == o.flops_unsharded(h, F, S)
        assert all(p * D == o.flops_unsharded(h, F, S) for p in per)
    # the 64K workload's figure from the closed form 8Th^2 + 6ThF + 4h(C^2(2D-1) + C(C+1))
    T, C = 8192, 4096
    assert o.flops_rank(4096, 11008, 65536, 8, 3) == (8 * T * 4096 ** 2 + 6 * T * 4096 * 11008
                                                      + 4 * 4096 * (C * C * 15 + C * (C + 1)))


ALL_PINS = [pin_zigzag_statement, pin_zigzag_partition, pin_zigzag_balance, pin_unzigzag,
            pin_rmsnorm_torch, pin_silu_torch, pin_attention_torch, pin_attention_loops,
            pin_attention_special, pin_layer_torch, pin_mlp_zero_gate, pin_fold_bruteforce,
            pin_mlp_partials, pin_stack, pin_flops]
