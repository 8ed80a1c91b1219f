"""GPU parity of the whole layer's backward (tsp_layer_shard_backward, the
dK/dV exchange tsp_kv_grad_reduce, tsp_layer_shard_backward_finish) against
the backward oracle's rank-by-rank replay (oracle/tsp_oracle_bwd.py,
fold_schedule_backward): every rank's input gradient and its partial
gradient of every weight shard and both gains.

All D ranks run on the one GPU: each runs its forward attention half (x1,
which training keeps) and part 1; the exchange sums the D ranks' partial
K/V gradients at each rank's positions; each rank then runs part 2.  Bar:
relative Frobenius error <= 1e-2 per gradient tensor (bf16 workloads).

Two modes: part 1 recomputes each head group's forward attention, or takes
the attention output and softmax normalisers that tsp_attn_shard_save kept.
The saved mode also checks that its x1 equals tsp_attn_shard's bit for bit
and its attention output against the oracle's multi-head attention.
"""
import numpy as np
import pytest
import torch

import oracle.tsp_oracle as O
import oracle.tsp_oracle_bwd as OB
import synth
from folded_tensor_sequence_rank_amd import tsp
from gpu_harness import DEV, RankRun, f64, fill_kv, layer_dev, new_kv, rel_fro, say, to_dev, tol

pytestmark = pytest.mark.gpu


def _cfg(**kw):
    base = dict(name="bwd", hidden=512, n_heads=4, head_dim=128, ffn=688, seq=2048, fold=4,
                ranks=(0,), layers=1, dtype="bf16")
    base.update(kw)
    return synth.LayerConfig(**base)


CASES = {
    # 128-dim heads, zigzag chunks on 64-key tiles (C = 256)
    "d128_c256": _cfg(),
    # ragged chunks (C = 200), 64-dim heads, two query heads per K/V head, rotary embedding
    "d64_c200_gqa2_rope": _cfg(hidden=256, head_dim=64, ffn=512, seq=1600, n_kv_heads=2, fold=2,
                               rope_theta=10000.0, x_std=0.02, w_std=0.045),
    # two sequences per call, fold 2
    "d128_b2_fold2": _cfg(seq=1024, fold=2, batch=2),
    # the 7B shape (h 4096, 32 heads of 128, FFN 11008) at fold 8, S = 2048
    "7b_s2k_fold8": synth.get_config("7b_s16k").with_(seq=2048),
}


_ORACLE = {}


def _oracle_bwd(case, cfg, xf, w, gf, b):
    """fold_schedule_backward of sequence b (both modes share it)."""
    key = (case, b)
    if key not in _ORACLE:
        _ORACLE[key] = OB.fold_schedule_backward(xf[b], w, cfg.n_heads, cfg.eps, gf[b], cfg.fold, cfg.rope_theta)
    return _ORACLE[key]


def _ws(dims, which):
    return torch.empty(max(tsp.workspace_bytes(dims, which), 256), dtype=torch.uint8, device=DEV)


def _cmp(cfg, name, got, want, worst):
    e = rel_fro(got, want)
    if e > worst[0]:
        worst[0], worst[1] = e, name
    assert np.isfinite(e) and e <= tol(cfg), f"{name}: rel {e:.3e}"


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_layer_backward_all_ranks(case, saved):
    cfg = CASES[case]
    D, B, S, h, H, d = cfg.fold, cfg.batch, cfg.seq, cfg.hidden, cfg.n_heads, cfg.head_dim
    T, BT = cfg.local_tokens, cfg.batch * cfg.local_tokens
    hs, Fs = h // D, cfg.ffn // D
    ks = cfg.kv_heads * d // D
    say(f"[gpu] layer backward {case} ({'saved attention' if saved else 'recomputed attention'}): h={h} H={H} Hkv={cfg.kv_heads} d={d} S={S} D={D} B={B} "
        f"theta={cfg.rope_theta}")
    w = synth.gen_weights(cfg)
    L = layer_dev(cfg, w)
    xf = [synth.gen_x_rows(cfg, 0, S, seq_index=b) for b in range(B)]
    gf = [synth.gen_x_rows(cfg, 0, S, layer=7, seq_index=b) for b in range(B)]  # output gradients
    pos = [O.zigzag_positions(S, D, r) for r in range(D)]
    xs = [to_dev(np.concatenate([x[p] for x in xf]), cfg) for p in pos]
    gs = [to_dev(np.concatenate([g[p] for g in gf]), cfg) for p in pos]
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    f32 = dict(dtype=torch.float32, device=DEV)
    outs = []
    a_worst = 0.0
    for r in range(D):  # forward attention half, then part 1
        dims = tsp.make_dims(cfg, r)
        run = RankRun(cfg, r)
        x1 = run.attn(xs[r], L, kv)
        a_saved = lse = None
        if saved:
            x1s, a_saved, lse = run.attn_save(xs[r], L, kv)
            assert torch.equal(x1s, x1), f"rank {r}: tsp_attn_shard_save's x1 differs from tsp_attn_shard's"
            if B == 1:  # the kept attention output against the oracle's
                n1 = O.rmsnorm(xf[0], w.g1, cfg.eps)
                a_ref = O.multihead_causal(n1, pos[r], w, H, cfg.rope_theta)
                e = rel_fro(f64(a_saved), a_ref)
                a_worst = max(a_worst, e)
                assert np.isfinite(e) and e <= tol(cfg), f"rank {r} saved attention output: rel {e:.3e}"
        o = dict(x1=x1, dx1=torch.empty_like(x1), dg2=torch.empty(h, **f32),
                 dw_mlp=[torch.empty(3 * Fs * h, **f32) for _ in range(D)],
                 dw_o=[torch.empty(h * hs, **f32) for _ in range(D)],
                 dq=torch.empty(H * BT * d, **f32), dkv=torch.full((2 * cfg.kv_heads * B * S * d,), float("nan"), **f32))
        tsp.tsp_layer_shard_backward(dims, xs[r], x1, L.g1, L.w_attn, kv, L.g2, L.w_mlp, gs[r], o["dx1"],
                                     o["dg2"], o["dw_mlp"], o["dw_o"], o["dq"], o["dkv"],
                                     _ws(dims, tsp.TSP_WS_LAYER_BWD), attn_saved=a_saved, lse_saved=lse)
        outs.append(o)
    for r in range(D):  # the exchange, then part 2
        dims = tsp.make_dims(cfg, r)
        o = outs[r]
        o["dkv_own"] = torch.empty(2 * cfg.kv_heads * BT * d, **f32)
        tsp.tsp_kv_grad_reduce(dims, [outs[q]["dkv"] for q in range(D)], o["dkv_own"])
        o["dx"] = torch.empty_like(xs[r])
        o["dg1"] = torch.empty(h, **f32)
        o["dw_qkv"] = [torch.empty((hs + 2 * ks) * h, **f32) for _ in range(D)]
        tsp.tsp_layer_shard_backward_finish(dims, xs[r], L.g1, L.w_attn, o["dx1"], o["dq"], o["dkv_own"], o["dx"],
                                            o["dg1"], o["dw_qkv"], _ws(dims, tsp.TSP_WS_LAYER_BWD_FINISH))
    torch.cuda.synchronize()
    say("    GPU done; oracle running")
    worst = [0.0, ""]
    for b in range(B):
        dx_ref, parts = _oracle_bwd(case, cfg, xf, w, gf, b)
        for r in range(D):
            o = outs[r]
            rows = slice(b * T, (b + 1) * T)
            _cmp(cfg, f"rank {r} seq {b} dx", f64(o["dx"])[rows], dx_ref[r], worst)
            if B > 1:
                continue  # weight gradients sum over the sequences: checked below
            _check_weights(cfg, r, o, parts[r], worst)
    if B > 1:  # partial weight gradients of each rank sum over its sequences
        refs = [_oracle_bwd(case, cfg, xf, w, gf, b)[1] for b in range(B)]
        for r in range(D):
            summed = OB.sum_partials([refs[b][r] for b in range(B)])
            _check_weights(cfg, r, outs[r], summed, worst)
    say(f"    {D} ranks: dx, dg1, dg2 and every shard's partial dW_Q/K/V/O/1/3/2 within {tol(cfg)}; "
        f"worst rel {worst[0]:.3e} ({worst[1]})" + (f"; saved A worst rel {a_worst:.3e}" if saved else ""))


def _check_weights(cfg, r, o, p, worst):
    D, h, d = cfg.fold, cfg.hidden, cfg.head_dim
    hs, Fs, ks = h // D, cfg.ffn // D, cfg.kv_heads * d // D
    _cmp(cfg, f"rank {r} dg1", f64(o["dg1"]), p.g1, worst)
    _cmp(cfg, f"rank {r} dg2", f64(o["dg2"]), p.g2, worst)
    for j in range(D):
        c, kc, fc = slice(j * hs, (j + 1) * hs), slice(j * ks, (j + 1) * ks), slice(j * Fs, (j + 1) * Fs)
        qkv = f64(o["dw_qkv"][j]).reshape(hs + 2 * ks, h)
        _cmp(cfg, f"rank {r} shard {j} dW_Q", qkv[:hs], p.wq[:, c].T, worst)
        _cmp(cfg, f"rank {r} shard {j} dW_K", qkv[hs:hs + ks], p.wk[:, kc].T, worst)
        _cmp(cfg, f"rank {r} shard {j} dW_V", qkv[hs + ks:], p.wv[:, kc].T, worst)
        _cmp(cfg, f"rank {r} shard {j} dW_O", f64(o["dw_o"][j]).reshape(h, hs), p.wo[c, :].T, worst)
        m = f64(o["dw_mlp"][j])
        _cmp(cfg, f"rank {r} shard {j} dW1", m[:Fs * h].reshape(Fs, h), p.w1[:, fc].T, worst)
        _cmp(cfg, f"rank {r} shard {j} dW3", m[Fs * h:2 * Fs * h].reshape(Fs, h), p.w3[:, fc].T, worst)
        _cmp(cfg, f"rank {r} shard {j} dW2", m[2 * Fs * h:].reshape(h, Fs), p.w2[fc, :].T, worst)
