"""GPU parity of the MLP half's backward (tsp_mlp_shard_backward) against the
backward oracle on the same rank's rows: the input gradient, this rank's
partial gradient of the norm gain, and its partial gradient of every weight
shard (unpacked from the shard layout)."""
import numpy as np
import pytest
import torch

import oracle.tsp_oracle as O
import oracle.tsp_oracle_bwd as B
import synth
from folded_tensor_sequence_rank_amd import tsp
from gpu_harness import DEV, f64, layer_dev, rel_fro, say, to_dev, tol
from test_gpu_parity import _check as _delta_check

pytestmark = pytest.mark.gpu


def _cfg(**kw):
    base = dict(name="case", hidden=512, n_heads=4, head_dim=128, ffn=1376, seq=2048, fold=4,
                ranks=(1,), layers=1, dtype="bf16")
    base.update(kw)
    return synth.LayerConfig(**base)


CASES = {
    "tiny_fp32": synth.get_config("tiny_fp32"),
    "bf16_h512_fold4": _cfg(gamma="normal"),
    "bf16_ragged_fs": _cfg(hidden=256, n_heads=4, head_dim=64, ffn=688, seq=1600, fold=4),  # F/D = 172, C = 200
    "f32_d64_fold2_b2": _cfg(hidden=128, n_heads=2, head_dim=64, ffn=344, seq=512, fold=2, dtype="f32",
                             batch=2),
    "7b_s16k_rank3": synth.get_config("7b_s16k"),
}


def _check(cfg, name, got, want):
    e = rel_fro(got, want)
    say(f"    {name}: rel {e:.3e} (bar {tol(cfg)})")
    assert np.isfinite(e) and e <= tol(cfg), (name, e)


@pytest.mark.parametrize("case", sorted(CASES))
def test_mlp_backward(case):
    cfg = CASES[case]
    r, D, h, Fs = cfg.ranks[0], cfg.fold, cfg.hidden, cfg.ffn // cfg.fold
    say(f"[gpu] MLP backward {case}: h={h} F={cfg.ffn} S={cfg.seq} D={D} B={cfg.batch} rank {r} {cfg.dtype}")
    w = synth.gen_weights(cfg)
    L = layer_dev(cfg, w)
    pos = O.zigzag_positions(cfg.seq, D, r)
    # x1 and the output gradient: seeded synthetic rows of each sequence
    x1 = np.concatenate([synth.gen_rows(cfg, pos, seq_index=b) for b in range(cfg.batch)])
    dout = np.concatenate([synth.gen_rows(cfg, pos, layer=7, seq_index=b) for b in range(cfg.batch)])
    x1_d, dout_d = to_dev(x1, cfg), to_dev(dout, cfg)
    x1, dout = f64(x1_d), f64(dout_d)  # the values the GPU receives
    dims = tsp.make_dims(cfg, r)
    ws = torch.empty(max(tsp.workspace_bytes(dims, tsp.TSP_WS_MLP_BWD), 256), dtype=torch.uint8, device=DEV)
    dx1 = torch.empty_like(x1_d)
    dg2 = torch.full((h,), float("nan"), dtype=torch.float32, device=DEV)
    dw = [torch.full((3 * Fs * h,), float("nan"), dtype=torch.float32, device=DEV) for _ in range(D)]
    tsp.tsp_mlp_shard_backward(dims, x1_d, L.g2, L.w_mlp, dout_d, dx1, dg2, dw, ws)
    torch.cuda.synchronize()
    say("    GPU done; oracle running")
    g2 = np.asarray(w.g2, np.float64)
    n2 = O.rmsnorm(x1, g2, cfg.eps)
    dn2 = np.zeros_like(n2)
    for j in range(D):
        c = slice(j * Fs, (j + 1) * Fs)
        dn, dw1, dw3, dw2 = B.swiglu_backward(n2, w.w1[:, c], w.w3[:, c], w.w2[c, :], dout)
        dn2 += dn
        got = f64(dw[j])
        _check(cfg, f"shard {j} dW1 (partial)", got[:Fs * h].reshape(Fs, h), dw1.T)
        _check(cfg, f"shard {j} dW3 (partial)", got[Fs * h:2 * Fs * h].reshape(Fs, h), dw3.T)
        _check(cfg, f"shard {j} dW2 (partial)", got[2 * Fs * h:].reshape(h, Fs), dw2.T)
    dxn, dg = B.rmsnorm_backward(x1, g2, cfg.eps, dn2)
    # whole output, and the MLP branch (dx1 - dout) beyond dx1's own storage
    # rounding, as for the forward blocks
    _delta_check(cfg, "dx1", f64(dx1), dout + dxn, dout, dout)
    _check(cfg, "dg2 (partial)", f64(dg2), dg)
    # the path sums in a fixed order (no atomics): a second call on the same
    # inputs gives the same bits
    dx1b, dg2b = torch.empty_like(dx1), torch.full_like(dg2, float("nan"))
    dwb = [torch.full_like(t, float("nan")) for t in dw]
    tsp.tsp_mlp_shard_backward(dims, x1_d, L.g2, L.w_mlp, dout_d, dx1b, dg2b, dwb, ws)
    torch.cuda.synchronize()
    assert torch.equal(dx1b, dx1) and torch.equal(dg2b, dg2), "second call differs"
    assert all(torch.equal(a_, b_) for a_, b_ in zip(dwb, dw)), "second call's weight gradients differ"


def test_mlp_backward_7b_s64k_rank3():
    """The MLP half's backward at the full 64K shape the layer-backward
    benchmark times (7B, S = 65536, fold 8, rank 3, 8192 rows).  A row's
    dx1 depends on that row alone, so it is checked on sampled rows; an
    intermediate column f's weight gradients (row f of a shard's dW1 / dW3,
    column f of its dW2) need that column's activations over all rows only,
    so they are checked on four sampled columns of every shard."""
    cfg = synth.get_config("7b_s64k")
    r, D, h, F = cfg.ranks[0], cfg.fold, cfg.hidden, cfg.ffn
    Fs = F // D
    say(f"[gpu] MLP backward 7b_s64k: h={h} F={F} S={cfg.seq} D={D} rank {r}")
    w = synth.gen_weights(cfg)
    L = layer_dev(cfg, w)
    pos = O.zigzag_positions(cfg.seq, D, r)
    x1_d = to_dev(synth.gen_rows(cfg, pos), cfg)
    dout_d = to_dev(synth.gen_rows(cfg, pos, layer=7), cfg)
    dims = tsp.make_dims(cfg, r)
    ws = torch.empty(tsp.workspace_bytes(dims, tsp.TSP_WS_MLP_BWD), dtype=torch.uint8, device=DEV)
    dx1 = torch.empty_like(x1_d)
    dg2 = torch.full((h,), float("nan"), dtype=torch.float32, device=DEV)
    dw = [torch.full((3 * Fs * h,), float("nan"), dtype=torch.float32, device=DEV) for _ in range(D)]
    tsp.tsp_mlp_shard_backward(dims, x1_d, L.g2, L.w_mlp, dout_d, dx1, dg2, dw, ws)
    torch.cuda.synchronize()
    say("    GPU done; oracle running")
    x1, dout = f64(x1_d), f64(dout_d)  # the values the GPU received
    T = x1.shape[0]
    g2 = np.asarray(w.g2, np.float64)
    rng = np.random.default_rng(77)
    # both chunks' edges and interior rows
    rows = np.unique(np.concatenate([[0, 1, T // 2 - 1, T // 2, T - 1], rng.integers(0, T, 43)]))
    n2r = O.rmsnorm(x1[rows], g2, cfg.eps)
    dn2r = B.swiglu_backward(n2r, w.w1, w.w3, w.w2, dout[rows])[0]
    dxn, _ = B.rmsnorm_backward(x1[rows], g2, cfg.eps, dn2r)
    _delta_check(cfg, f"dx1 on {rows.size} rows", f64(dx1)[rows], dout[rows] + dxn, dout[rows], dout[rows])
    # four intermediate columns of every shard: its first, its last, two inside
    local = [np.unique(np.concatenate([[0, Fs - 1], rng.integers(1, Fs - 1, 2)])) for _ in range(D)]
    cols = np.concatenate([j * Fs + local[j] for j in range(D)])
    n2 = O.rmsnorm(x1, g2, cfg.eps)
    _, ew1, ew3, ew2 = B.swiglu_backward(n2, w.w1[:, cols], w.w3[:, cols], w.w2[cols, :], dout)
    at = 0
    for j in range(D):
        k = local[j].size
        got = f64(dw[j])
        _check(cfg, f"shard {j} dW1 rows {[int(v) for v in local[j]]}", got[:Fs * h].reshape(Fs, h)[local[j]],
               ew1[:, at:at + k].T)
        _check(cfg, f"shard {j} dW3 rows", got[Fs * h:2 * Fs * h].reshape(Fs, h)[local[j]], ew3[:, at:at + k].T)
        _check(cfg, f"shard {j} dW2 columns", got[2 * Fs * h:].reshape(h, Fs)[:, local[j]], ew2[at:at + k].T)
        at += k
