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
  * for the extensions the pages do not describe (rotary embedding,
    grouped-query attention): the Llama decoder layer and rotary embedding of
    the transformers library, in float64 on the CPU (its rotary angles are
    formed in float32, hence the 1e-4 bounds at small positions); torch's
    scaled_dot_product_attention with enable_gqa; and the relative-position
    property of rotated dot products.
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


def _rel(got, want):
    """Relative Frobenius distance, written out here so that no pin grades the
    oracle with the oracle's own norm."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return math.sqrt(float(((got - want) ** 2).sum())) / max(math.sqrt(float((want ** 2).sum())), 1e-300)


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
        assert _rel(got, want) < 1e-12, _rel(got, want)
        # restricted rows, the attention half and the MLP half agree too
        rows = o.zigzag_positions(cfg.seq, cfg.fold, 1)
        assert _rel(o.layer_rows(x, w, cfg.n_heads, cfg.eps, rows), want[rows]) < 1e-12
        x1 = o.attention_block_rows(x, w, cfg.n_heads, cfg.eps, np.arange(cfg.seq))
        assert _rel(o.mlp_block(x1, w, cfg.eps), want) < 1e-12
        assert _rel(o.rank_share(x, w, cfg.n_heads, cfg.eps, cfg.seq, cfg.fold, 1),
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
        assert _rel(o.unzigzag(parts, cfg.seq, cfg.fold), want) < 1e-12, cfg


def pin_mlp_partials(o):
    """Partial MLP outputs of the D shards sum to the full MLP (no all-reduce)."""
    for cfg in [TINY, TINY.with_(ffn=176, fold=8), TINY.with_(fold=1)]:
        w = _weights(cfg)
        n = _rng(5).standard_normal((33, cfg.hidden))
        full = o.swiglu_mlp(n, w.w1, w.w3, w.w2)
        parts = o.mlp_partials(n, w, cfg.fold)
        assert len(parts) == cfg.fold
        assert _rel(sum(parts), full) < 1e-13


def pin_stack(o):
    cfg = TINY.with_(layers=2, seq=64, fold=2)
    ws = [_weights(cfg, l) for l in range(2)]
    x = _x(cfg)
    want = torch_layer(torch_layer(x, ws[0], cfg.n_heads, cfg.eps), ws[1], cfg.n_heads, cfg.eps)
    rows = np.array([0, 5, 17, 63])
    assert _rel(o.stack_rows(x, ws, cfg.n_heads, cfg.eps, rows), want[rows]) < 1e-12


# ---------------------------------------------------------------- rotary embedding, GQA

def _llama():
    from transformers import LlamaConfig
    from transformers.models.llama import modeling_llama as ml
    return LlamaConfig, ml


def _half_split(d):
    """Dim order of the Llama rotary convention (pairs (i, i + d/2)) in terms
    of the RoFormer order (pairs (2i, 2i+1)): Llama dim i is RoFormer dim
    2i, Llama dim d/2 + i is RoFormer dim 2i + 1."""
    return np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])


def pin_rope_llama(o):
    LlamaConfig, ml = _llama()
    for d, theta in [(16, 10000.0), (128, 10000.0), (8, 500.0)]:
        cfg = LlamaConfig(hidden_size=d, num_attention_heads=1, num_key_value_heads=1, head_dim=d,
                          rope_theta=theta, max_position_embeddings=1024)
        rot = ml.LlamaRotaryEmbedding(cfg).double()
        pos = np.array([0, 1, 2, 3, 7, 31, 64, 100, 255])
        x = _rng(11).standard_normal((pos.size, d))
        P = _half_split(d)
        xt = torch.from_numpy(x[:, P])[None, None]          # [1, 1, R, d]
        cos, sin = rot(xt[0], torch.from_numpy(pos)[None])
        want, _ = ml.apply_rotary_pos_emb(xt, xt, cos, sin)
        got = o.rope(x, pos, theta)[:, P]
        err = np.abs(got - want[0, 0].numpy()).max()
        assert err < 1e-4, (d, theta, err)
        assert np.array_equal(o.rope(x, pos, 0.0), x)


def pin_rope_relative(o):
    """Rotated dot products depend on the position difference only; rows at
    position 0 are unchanged; each pair keeps its length."""
    rng = _rng(12)
    d = 16
    q, k = rng.standard_normal((2, 1, d))
    for theta in (10000.0, 50.0):
        for m, n, c in [(5, 3, 0), (5, 3, 17), (0, 9, 1000), (40000, 39990, 90000)]:
            a = o.rope(q, [m], theta) @ o.rope(k, [n], theta).T
            b = o.rope(q, [m + c], theta) @ o.rope(k, [n + c], theta).T
            assert abs(a - b).max() < 1e-9 * (1 + abs(a).max()), (theta, m, n, c)
        r = o.rope(q, [123], theta)
        assert np.allclose(r[:, 0::2] ** 2 + r[:, 1::2] ** 2, q[:, 0::2] ** 2 + q[:, 1::2] ** 2)
        assert np.array_equal(o.rope(q, [0], theta), q)
        # the lowest pair turns by exactly the position (in radians), counter-clockwise
        e = np.zeros((1, d)); e[0, 0] = 1.0
        assert np.allclose(o.rope(e, [1], theta)[0, :2], [math.cos(1.0), math.sin(1.0)], atol=1e-15)


def _gqa(cfg, hkv, theta=0.0):
    return cfg.with_(n_kv_heads=hkv, rope_theta=theta)


def pin_gqa_torch(o):
    """Grouped-query attention against torch's enable_gqa attention, by way of
    the torch layer composition (no rotary embedding)."""
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    for cfg in [_gqa(TINY, 2), _gqa(TINY, 1), _gqa(TINY.with_(n_heads=8, head_dim=8), 4)]:
        w, x = _weights(cfg), _x(cfg)
        H, h, d, hkv = cfg.n_heads, cfg.hidden, cfg.head_dim, cfg.n_kv_heads
        assert o.kv_heads(w, H) == hkv
        X = T(x)
        S = X.shape[0]
        n1 = Fn.rms_norm(X, (h,), weight=T(w.g1), eps=cfg.eps)
        heads = lambda m, nh: (n1 @ T(m)).reshape(S, nh, d).transpose(0, 1).contiguous()
        a = Fn.scaled_dot_product_attention(heads(w.wq, H), heads(w.wk, hkv), heads(w.wv, hkv),
                                            is_causal=True, enable_gqa=True)
        want = (X + a.transpose(0, 1).reshape(S, h) @ T(w.wo)).numpy()
        got = o.attention_block_rows(x, w, H, cfg.eps, np.arange(S))
        assert _rel(got, want) < 1e-12, (cfg.n_heads, hkv, _rel(got, want))


def llama_layer(x, w, cfg):
    """The layer as transformers' Llama decoder layer (float64, CPU), the
    oracle's weights loaded into it with Q and K columns put in its rotary
    dim order."""
    LlamaConfig, ml = _llama()
    H, d, hkv = cfg.n_heads, cfg.head_dim, cfg.kv_heads
    lc = LlamaConfig(hidden_size=cfg.hidden, num_attention_heads=H, num_key_value_heads=hkv,
                     head_dim=d, intermediate_size=cfg.ffn, rms_norm_eps=cfg.eps,
                     rope_theta=cfg.rope_theta, max_position_embeddings=max(2048, cfg.seq),
                     attention_bias=False, mlp_bias=False)
    lc._attn_implementation = "eager"
    layer = ml.LlamaDecoderLayer(lc, layer_idx=0).double().eval()
    rot = ml.LlamaRotaryEmbedding(lc).double()
    P = _half_split(d)
    cols = lambda nh: np.concatenate([t * d + P for t in range(nh)])
    T = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float64)))
    sd = {"self_attn.q_proj.weight": T(w.wq[:, cols(H)].T), "self_attn.k_proj.weight": T(w.wk[:, cols(hkv)].T),
          "self_attn.v_proj.weight": T(w.wv.T), "self_attn.o_proj.weight": T(w.wo.T),
          "mlp.gate_proj.weight": T(w.w1.T), "mlp.up_proj.weight": T(w.w3.T),
          "mlp.down_proj.weight": T(w.w2.T), "input_layernorm.weight": T(w.g1),
          "post_attention_layernorm.weight": T(w.g2)}
    layer.load_state_dict(sd)
    X = T(x)[None]
    pos = torch.arange(X.shape[1])[None]
    S = X.shape[1]
    mask = torch.full((S, S), -math.inf, dtype=torch.float64).triu(1)[None, None]
    with torch.no_grad():
        out = layer(X, attention_mask=mask, position_ids=pos, position_embeddings=rot(X, pos))
    return (out[0] if isinstance(out, tuple) else out)[0].numpy()


def pin_layer_llama(o):
    """Rotary embedding and grouped-query attention in the whole layer."""
    # weights of std 0.2 make the attention sharp enough that the rotation
    # changes the output by O(1) (checked below), so a wrong angle shows
    base = TINY.with_(seq=64, fold=2, w_std=0.2)
    for cfg in [_gqa(base, 2, 10000.0), _gqa(base, 4, 100.0), _gqa(base, 1, 10000.0),
                _gqa(base.with_(hidden=64, n_heads=2, head_dim=32), 2, 10000.0)]:
        w, x = _weights(cfg), _x(cfg)
        want = llama_layer(x, w, cfg)
        got = o.layer_unsharded(x, w, cfg.n_heads, cfg.eps, cfg.rope_theta)
        assert _rel(got, want) < 1e-5, (cfg.n_kv_heads, cfg.rope_theta, _rel(got, want))
    cfg = _gqa(base, 2, 10000.0)
    w, x = _weights(cfg), _x(cfg)
    assert _rel(o.layer_unsharded(x, w, cfg.n_heads, cfg.eps, 0.0), llama_layer(x, w, cfg)) > 0.1


def pin_fold_rope_gqa(o):
    """The literal D-rank schedule with the rotary embedding applied at the
    ranks' global (zigzag) positions, and grouped K/V shards, equals the
    unsharded layer."""
    base = TINY.with_(seq=64, w_std=0.2)
    for cfg in [_gqa(base.with_(fold=2), 2, 10000.0), _gqa(base, 4, 100.0),
                _gqa(base.with_(fold=2, n_heads=8, head_dim=8), 2, 10000.0)]:
        w, x = _weights(cfg), _x(cfg)
        want = o.layer_unsharded(x, w, cfg.n_heads, cfg.eps, cfg.rope_theta)
        parts = o.fold_schedule(x, w, cfg.n_heads, cfg.eps, cfg.fold, rope_theta=cfg.rope_theta)
        assert _rel(o.unzigzag(parts, cfg.seq, cfg.fold), want) < 1e-12, cfg
        r = cfg.fold - 1
        got = o.rank_share(x, w, cfg.n_heads, cfg.eps, cfg.seq, cfg.fold, r, cfg.rope_theta)
        assert _rel(got, parts[r]) < 1e-12


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
            pin_mlp_partials, pin_stack, pin_flops, pin_rope_llama, pin_rope_relative,
            pin_gqa_torch, pin_layer_llama, pin_fold_rope_gqa]
