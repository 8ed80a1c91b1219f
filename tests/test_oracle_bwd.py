"""The backward oracle against its pins, and the pins against planted mistakes.

Pins: torch autograd in float64 (rms_norm, the SwiGLU MLP, causal
scaled_dot_product_attention, the torch composition of the whole layer);
autograd through transformers' Llama decoder layer for the rotary embedding
and grouped K/V heads; a central finite difference of the layer that uses no
library; and the per-rank reading replayed rank by rank against the unsharded
gradients (un-zigzagged input gradients, summed weight partials).
"""
import ast
import math
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle.tsp_oracle as O
import oracle.tsp_oracle_bwd as B
import synth
from oracle_pins import TINY, _gqa, _half_split, _llama, _weights, _x, torch_layer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
T64 = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float64)))
rel = O.rel_fro


def _dout(shape, seed=21):
    return np.random.default_rng(seed).standard_normal(shape)


def pin_rmsnorm_torch(b):
    x = np.random.default_rng(1).standard_normal((7, 48)) * 3
    g = 1 + 0.1 * np.random.default_rng(2).standard_normal(48)
    dy = _dout((7, 48))
    X, G = T64(x).requires_grad_(), T64(g).requires_grad_()
    Fn.rms_norm(X, (48,), weight=G, eps=1e-5).backward(T64(dy))
    dx, dg = b.rmsnorm_backward(x, g, 1e-5, dy)
    assert rel(dx, X.grad.numpy()) < 1e-12 and rel(dg, G.grad.numpy()) < 1e-12


def pin_swiglu_torch(b):
    rng = np.random.default_rng(3)
    n, w1, w3, w2 = (rng.standard_normal(s) * c for s, c in
                     (((9, 16), 1), ((16, 24), 0.5), ((16, 24), 0.5), ((24, 16), 0.5)))
    dout = _dout((9, 16))
    N, W1, W3, W2 = (T64(t).requires_grad_() for t in (n, w1, w3, w2))
    ((Fn.silu(N @ W1) * (N @ W3)) @ W2).backward(T64(dout))
    got = b.swiglu_backward(n, w1, w3, w2, dout)
    for g, t in zip(got, (N, W1, W3, W2)):
        assert rel(g, t.grad.numpy()) < 1e-12


def pin_attention_torch(b):
    rng = np.random.default_rng(4)
    for S, d in ((1, 8), (13, 16), (70, 32)):
        q, k, v = (rng.standard_normal((S, d)) for _ in range(3))
        do = _dout((S, d))
        Q, K, V = (T64(t).requires_grad_() for t in (q, k, v))
        Fn.scaled_dot_product_attention(Q[None], K[None], V[None], is_causal=True)[0].backward(T64(do))
        dq, dk, dv = b.causal_attention_backward(q, np.arange(S), k, v, do)
        assert rel(dq, Q.grad.numpy()) < 1e-11 and rel(dk, K.grad.numpy()) < 1e-11
        assert rel(dv, V.grad.numpy()) < 1e-11


def _layer_params(w):
    return {k: T64(getattr(w, k)).requires_grad_() for k in ("g1", "wq", "wk", "wv", "wo", "g2", "w1", "w3", "w2")}


def pin_layer_torch(b):
    """MHA, no rotary embedding: the torch composition of the layer, autograd."""
    for cfg in (TINY.with_(seq=64, fold=2), TINY.with_(seq=32, fold=2, w_std=0.2)):
        w, x = _weights(cfg), _x(cfg)
        dout = _dout(x.shape)
        P = _layer_params(w)
        X = T64(x).requires_grad_()
        H, h = cfg.n_heads, cfg.hidden
        d = h // H
        S = x.shape[0]
        n1 = Fn.rms_norm(X, (h,), weight=P["g1"], eps=cfg.eps)
        heads = lambda m: (n1 @ m).reshape(S, H, d).transpose(0, 1).contiguous()
        a = Fn.scaled_dot_product_attention(heads(P["wq"]), heads(P["wk"]), heads(P["wv"]), is_causal=True)
        x1 = X + a.transpose(0, 1).reshape(S, h) @ P["wo"]
        n2 = Fn.rms_norm(x1, (h,), weight=P["g2"], eps=cfg.eps)
        out = x1 + (Fn.silu(n2 @ P["w1"]) * (n2 @ P["w3"])) @ P["w2"]
        assert rel(out.detach().numpy(), torch_layer(x, w, H, cfg.eps)) < 1e-12
        out.backward(T64(dout))
        dx, g = b.layer_backward(x, w, H, cfg.eps, dout)
        assert rel(dx, X.grad.numpy()) < 1e-10, rel(dx, X.grad.numpy())
        for k, t in P.items():
            assert rel(getattr(g, k), t.grad.numpy()) < 1e-10, (k, rel(getattr(g, k), t.grad.numpy()))


def pin_layer_llama(b):
    """Rotary embedding and grouped K/V heads: autograd through transformers'
    Llama decoder layer in float64 (its rotary angles are float32, hence 1e-5)."""
    LlamaConfig, ml = _llama()
    base = TINY.with_(seq=48, fold=2, w_std=0.2)
    for cfg in (_gqa(base, 2, 10000.0), _gqa(base, 4, 100.0)):
        w, x = _weights(cfg), _x(cfg)
        dout = _dout(x.shape)
        H, d, hkv = cfg.n_heads, cfg.head_dim, cfg.kv_heads
        lc = LlamaConfig(hidden_size=cfg.hidden, num_attention_heads=H, num_key_value_heads=hkv,
                         head_dim=d, intermediate_size=cfg.ffn, rms_norm_eps=cfg.eps,
                         rope_theta=cfg.rope_theta, max_position_embeddings=2048,
                         attention_bias=False, mlp_bias=False)
        lc._attn_implementation = "eager"
        layer = ml.LlamaDecoderLayer(lc, layer_idx=0).double()
        rot = ml.LlamaRotaryEmbedding(lc).double()
        perm = _half_split(d)
        cols = lambda nh: np.concatenate([t * d + perm for t in range(nh)])
        sd = {"self_attn.q_proj.weight": T64(w.wq[:, cols(H)].T), "self_attn.k_proj.weight": T64(w.wk[:, cols(hkv)].T),
              "self_attn.v_proj.weight": T64(w.wv.T), "self_attn.o_proj.weight": T64(w.wo.T),
              "mlp.gate_proj.weight": T64(w.w1.T), "mlp.up_proj.weight": T64(w.w3.T),
              "mlp.down_proj.weight": T64(w.w2.T), "input_layernorm.weight": T64(w.g1),
              "post_attention_layernorm.weight": T64(w.g2)}
        layer.load_state_dict(sd)
        X = T64(x)[None].requires_grad_()
        S = x.shape[0]
        posi = torch.arange(S)[None]
        mask = torch.full((S, S), -math.inf, dtype=torch.float64).triu(1)[None, None]
        out = layer(X, attention_mask=mask, position_ids=posi, position_embeddings=rot(X, posi))
        (out[0] if isinstance(out, tuple) else out).backward(T64(dout)[None])
        dx, g = b.layer_backward(x, w, H, cfg.eps, dout, cfg.rope_theta)
        assert rel(dx, X.grad[0].numpy()) < 1e-5, rel(dx, X.grad[0].numpy())
        pr = dict(layer.named_parameters())
        inv = lambda nh: np.argsort(cols(nh))
        checks = {"wq": pr["self_attn.q_proj.weight"].grad.numpy().T[:, inv(H)],
                  "wk": pr["self_attn.k_proj.weight"].grad.numpy().T[:, inv(hkv)],
                  "wv": pr["self_attn.v_proj.weight"].grad.numpy().T,
                  "wo": pr["self_attn.o_proj.weight"].grad.numpy().T,
                  "w1": pr["mlp.gate_proj.weight"].grad.numpy().T, "w3": pr["mlp.up_proj.weight"].grad.numpy().T,
                  "w2": pr["mlp.down_proj.weight"].grad.numpy().T,
                  "g1": pr["input_layernorm.weight"].grad.numpy(), "g2": pr["post_attention_layernorm.weight"].grad.numpy()}
        for k, ref in checks.items():
            assert rel(getattr(g, k), ref) < 1e-5, (k, rel(getattr(g, k), ref))


def pin_finite_difference(b):
    """<dx, u> and <dW_K, U> against central differences of <out, dout>."""
    cfg = _gqa(TINY.with_(seq=24, fold=2, w_std=0.2), 2, 500.0)
    w, x = _weights(cfg), _x(cfg)
    dout = _dout(x.shape)
    f = lambda xx, ww: float(np.sum(O.layer_unsharded(xx, ww, cfg.n_heads, cfg.eps, cfg.rope_theta) * dout))
    dx, g = b.layer_backward(x, w, cfg.n_heads, cfg.eps, dout, cfg.rope_theta)
    rng = np.random.default_rng(9)
    u = rng.standard_normal(x.shape)
    e = 1e-5
    fd = (f(x + e * u, w) - f(x - e * u, w)) / (2 * e)
    assert abs(fd - np.sum(dx * u)) < 1e-6 * (1 + abs(fd)), (fd, np.sum(dx * u))
    U = rng.standard_normal(w.wk.shape)
    wp, wm = types.SimpleNamespace(**vars(w)), types.SimpleNamespace(**vars(w))
    wp.wk, wm.wk = w.wk + e * U, w.wk - e * U
    fd = (f(x, wp) - f(x, wm)) / (2 * e)
    assert abs(fd - np.sum(g.wk * U)) < 1e-6 * (1 + abs(fd)), (fd, np.sum(g.wk * U))


def pin_fold_schedule(b):
    """Each rank's rows and partial weight gradients, with dK/dV summed at
    their owners, rebuild the unsharded gradients."""
    base = TINY.with_(seq=64, w_std=0.2)
    for cfg in (base.with_(fold=1), base.with_(fold=2), base, _gqa(base.with_(fold=2), 2, 10000.0),
                _gqa(base, 4, 100.0)):
        w, x = _weights(cfg), _x(cfg)
        dout = _dout(x.shape)
        dx, g = b.layer_backward(x, w, cfg.n_heads, cfg.eps, dout, cfg.rope_theta)
        parts_dx, parts = b.fold_schedule_backward(x, w, cfg.n_heads, cfg.eps, dout, cfg.fold, cfg.rope_theta)
        assert rel(O.unzigzag(parts_dx, cfg.seq, cfg.fold), dx) < 1e-12
        tot = b.sum_partials(parts)
        for k in ("g1", "wq", "wk", "wv", "wo", "g2", "w1", "w3", "w2"):
            assert rel(getattr(tot, k), getattr(g, k)) < 1e-12, (cfg.fold, k)


BWD_PINS = [pin_rmsnorm_torch, pin_swiglu_torch, pin_attention_torch, pin_layer_torch,
            pin_layer_llama, pin_finite_difference, pin_fold_schedule]


@pytest.mark.parametrize("pin", BWD_PINS, ids=[p.__name__ for p in BWD_PINS])
def test_pin(pin):
    pin(B)


MUTATIONS = {
    "softmax_grad_no_rowsum": ("ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))", "ds = p * dp"),
    "silu_derivative_is_sigmoid": ("sg * (1.0 + a * (1.0 - sg))", "sg"),
    "rms_grad_no_norm_term": (" - x * r ** 3 * np.sum(u * x, axis=-1, keepdims=True) / h", ""),
    "no_residual_gradient": ("dx1 = dout + dx1n", "dx1 = dx1n"),
    "rope_grad_same_direction": ("dq_all[:, c] = rope(dq, -pos, rope_theta)",
                                 "dq_all[:, c] = rope(dq, pos, rope_theta)"),
    "gqa_grads_overwritten": ("dk_all[:, kc] += rope(dk, -pos, rope_theta)",
                              "dk_all[:, kc] = rope(dk, -pos, rope_theta)"),
    "kv_grads_not_reduced": ("dk_sum, dv_sum = dk_part.sum(axis=0), dv_part.sum(axis=0)",
                             "dk_sum, dv_sum = dk_part.max(axis=0), dv_part.sum(axis=0)"),
    "fold_rope_grad_same_direction": ("dqr[:, c] = rope(gq, -pos[r], rope_theta)",
                                      "dqr[:, c] = rope(gq, pos[r], rope_theta)"),
}


def _mutant(old, new):
    src = open(os.path.join(ROOT, "oracle", "tsp_oracle_bwd.py")).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    ast.parse(src)
    mod = types.ModuleType("tsp_oracle_bwd_mutant")
    exec(compile(src, "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    mutant = _mutant(*MUTATIONS[name])
    failed = []
    for pin in BWD_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutation {name}"
