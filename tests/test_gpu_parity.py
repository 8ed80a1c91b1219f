"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar (tests/parity.py): relative Frobenius error <= 1e-2 for bf16 workloads
and <= 1e-4 for fp32, on the whole output and on each block's delta (x1 - x,
out - x1), so the residual cannot hide an error; and twice that on every
(row, head-sized column block), so an error confined to one head of one
query tile cannot hide in the global norm.  The oracle runs in float64 on the
very values the GPU receives.
"""
import numpy as np
import pytest
import torch

import oracle.tsp_oracle as O
import synth
from gpu_harness import (LayerDev, RankRun, f64, fill_kv, layer_dev, new_kv, rel_fro, say,
                         to_dev, tol)
from parity import compare

pytestmark = pytest.mark.gpu

TINY = synth.get_config("tiny_fp32")


def _cfg(**kw):
    base = dict(name="case", hidden=256, n_heads=2, head_dim=128, ffn=688, seq=1600, fold=4,
                ranks=(0,), layers=1, dtype="bf16")
    base.update(kw)
    return synth.LayerConfig(**base)


# Small workloads that together cover several tiles and ragged tails in every
# dimension, each head size, fold 1/2/4/8, fp32 and bf16, a random RMSNorm
# gain, and chunk lengths that are not multiples of the 128-row query tile.
SMALL = {
    "tiny_fp32": TINY,
    "tiny_bf16": TINY.with_(dtype="bf16"),
    "bf16_d128_ragged": _cfg(hidden=512, n_heads=4),              # C=200, F/D=172
    # C=256: other ranks' K/V rows are read in place (C % 64 == 0)
    "bf16_d128_inplace": _cfg(hidden=512, n_heads=4, ffn=1376, seq=2048),
    "bf16_d128_ragged_lowres": _cfg(hidden=512, n_heads=4, x_std=0.02),
    "bf16_d64_lowres_gamma": _cfg(hidden=256, n_heads=4, head_dim=64, ffn=1024, seq=2048, fold=4,
                                  x_std=0.02, gamma="normal"),
    "tiny_bf16_lowres": TINY.with_(dtype="bf16", x_std=0.02),
    "bf16_d64_fold2": _cfg(hidden=256, n_heads=4, head_dim=64, ffn=512, seq=1024, fold=2),
    "bf16_d32_fold8_gamma": _cfg(hidden=256, n_heads=8, head_dim=32, ffn=704, seq=1024, fold=8,
                                 gamma="normal"),
    "bf16_d16_fold1": _cfg(hidden=64, n_heads=4, head_dim=16, ffn=176, seq=200, fold=1),
    "bf16_c20": _cfg(hidden=128, n_heads=4, head_dim=32, ffn=344, seq=160, fold=4),
    "f32_d64": _cfg(hidden=128, n_heads=2, head_dim=64, ffn=344, seq=512, fold=2, dtype="f32"),
    "f32_d128_fold4": _cfg(hidden=512, n_heads=4, head_dim=128, ffn=1376, seq=1024, fold=4,
                           dtype="f32", gamma="normal"),
}


def _setup(cfg, layer=0):
    w = synth.gen_weights(cfg, layer)
    x_full = synth.gen_x_rows(cfg, 0, cfg.seq, layer)
    L = layer_dev(cfg, w)
    pos = [O.zigzag_positions(cfg.seq, cfg.fold, r) for r in range(cfg.fold)]
    from folded_tensor_sequence_rank_amd import tsp
    for r in range(cfg.fold):  # the library's zigzag agrees with the oracle's
        assert np.array_equal(tsp.zigzag_positions(cfg.seq, cfg.fold, r), pos[r])
    xs = [to_dev(x_full[p], cfg) for p in pos]
    return w, x_full, L, xs, pos


def _check(cfg, name, got, want, base=None, want_base=None):
    """The parity bar of tests/parity.py: whole tensor and block delta within
    tol, every (row, head-sized column block) within 2 * tol (plus the output's
    storage rounding)."""
    ok, msg, _ = compare(cfg, got, want, base, want_base)
    say("   ", f"{name}: {msg}")
    assert ok, f"{name}: {msg}"


@pytest.mark.parametrize("case", sorted(SMALL))
def test_small_all_ranks(case):
    cfg = SMALL[case]
    say(f"[gpu] small parity {case}: h={cfg.hidden} H={cfg.n_heads} d={cfg.head_dim} "
        f"F={cfg.ffn} S={cfg.seq} D={cfg.fold} {cfg.dtype}")
    w, x_full, L, xs, pos = _setup(cfg)
    x1_ref = O.attention_block_rows(x_full, w, cfg.n_heads, cfg.eps, np.arange(cfg.seq))
    out_ref = O.mlp_block(x1_ref, w, cfg.eps)
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    parts = []
    for r in range(cfg.fold):
        run = RankRun(cfg, r)
        x1 = run.attn(xs[r], L, kv)
        out = run.mlp(x1, L)
        lay = run.layer(xs[r], L, kv)
        torch.cuda.synchronize()
        xr = x_full[pos[r]].astype(np.float64)
        _check(cfg, f"rank {r} x1", f64(x1), x1_ref[pos[r]], xr, xr)
        _check(cfg, f"rank {r} out", f64(out), out_ref[pos[r]], f64(x1), x1_ref[pos[r]])
        assert torch.equal(lay, out), "layer call differs from attention + MLP calls"
        parts.append(f64(lay))
    # brute force over the fold: un-zigzagged shares rebuild the unsharded layer
    full = O.unzigzag(parts, cfg.seq, cfg.fold)
    _check(cfg, "all ranks un-zigzagged", full, out_ref)


def test_split_attention_items():
    """A shape whose query tiles are split over several key segments and
    merged afterwards."""
    cfg = _cfg(hidden=512, n_heads=4, head_dim=128, ffn=1024, seq=8192, fold=2)
    say("[gpu] split-segment attention parity, S=8192 D=2")
    w, x_full, L, xs, pos = _setup(cfg)
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    for r in range(cfg.fold):
        x1 = RankRun(cfg, r).attn(xs[r], L, kv)
        torch.cuda.synchronize()
        ref = O.attention_block_rows(x_full, w, cfg.n_heads, cfg.eps, pos[r])
        xr = x_full[pos[r]].astype(np.float64)
        _check(cfg, f"rank {r} x1", f64(x1), ref, xr, xr)


@pytest.mark.parametrize("case", ["bf16_d128_ragged", "bf16_d128_inplace", "split"])
def test_softmax_rescale_path(case):
    """TSP_F_RESCALE_TEST lowers the bound at which the 128-dim bf16
    attention raises its lazy softmax reference from 2^64 to 2, so the rescale
    path (O, row sum and the P block already formed rescaled, the block
    redone) runs on most tiles; every rank must still match the oracle."""
    from folded_tensor_sequence_rank_amd import tsp
    cfg = (SMALL[case] if case != "split" else
           _cfg(hidden=512, n_heads=4, head_dim=128, ffn=1024, seq=8192, fold=2))
    say(f"[gpu] softmax rescale path ({case})")
    w, x_full, L, xs, pos = _setup(cfg)
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    for r in range(cfg.fold):
        x1 = RankRun(cfg, r, flags=tsp.TSP_F_RESCALE_TEST).attn(xs[r], L, kv)
        torch.cuda.synchronize()
        ref = O.attention_block_rows(x_full, w, cfg.n_heads, cfg.eps, pos[r])
        xr = x_full[pos[r]].astype(np.float64)
        _check(cfg, f"rank {r} x1", f64(x1), ref, xr, xr)


@pytest.mark.parametrize("case", ["bf16_d128_ragged", "bf16_d128_inplace"])
def test_own_kv_rows_not_read(case):
    """The rank's own rows in the gathered K/V stay NaN: it must use the rows
    it projects itself (other ranks' rows copied, C=200, or read in place,
    C=256)."""
    cfg = SMALL[case]
    say(f"[gpu] own K/V rows are computed, not read ({case})")
    w, x_full, L, xs, pos = _setup(cfg)
    r = 2
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv, skip=r)
    out = RankRun(cfg, r).layer(xs[r], L, kv)
    torch.cuda.synchronize()
    ref = O.layer_rows(x_full, w, cfg.n_heads, cfg.eps, pos[r])
    _check(cfg, "rank 2 out", f64(out), ref)


@pytest.mark.parametrize("flags", ["delay_poison", "no_overlap", "null_copy_stream"])
def test_stream_handoff_bitwise(flags):
    """Delaying the copy stream and poisoning slots with NaN before each
    refill must not change a single bit; neither must running the copies in
    order on the compute stream.  Repeated runs are bitwise reproducible."""
    from folded_tensor_sequence_rank_amd import tsp
    cfg = SMALL["bf16_d32_fold8_gamma"]
    say(f"[gpu] stream hand-off, mode {flags}")
    w, x_full, L, xs, pos = _setup(cfg)
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    r = 5
    base = RankRun(cfg, r).layer(xs[r], L, kv)
    again = RankRun(cfg, r).layer(xs[r], L, kv)
    if flags == "delay_poison":
        run = RankRun(cfg, r, flags=tsp.TSP_F_DELAY_COPY | tsp.TSP_F_POISON_SLOTS)
    elif flags == "no_overlap":
        run = RankRun(cfg, r, flags=tsp.TSP_F_NO_OVERLAP)
    else:
        run = RankRun(cfg, r, copy_stream=False)
    other = run.layer(xs[r], L, kv)
    other2 = run.layer(xs[r], L, kv)
    torch.cuda.synchronize()
    assert torch.equal(base, again)
    assert torch.equal(base, other)
    assert torch.equal(base, other2)
    assert torch.isfinite(other).all()


@pytest.mark.parametrize("case", ["bf16_d128_inplace", "bf16_d64_lowres_gamma"])
def test_kv_stream_flag_bitwise(case):
    """TSP_F_KV_STREAM copies the other ranks' K/V rows into the slot on the
    side stream even where chunks align with the 64-key tiles; the attention
    then reads every row from the slot.  Same values, same order: every rank's
    output must equal the in-place path bit for bit, also with delayed and
    NaN-poisoned copies."""
    from folded_tensor_sequence_rank_amd import tsp
    cfg = SMALL[case]
    assert cfg.chunk % 64 == 0
    say(f"[gpu] K/V all-gather through the shard stream ({case})")
    w, x_full, L, xs, pos = _setup(cfg)
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    for r in range(cfg.fold):
        base = RankRun(cfg, r).layer(xs[r], L, kv)
        streamed = RankRun(cfg, r, flags=tsp.TSP_F_KV_STREAM).layer(xs[r], L, kv)
        stressed = RankRun(cfg, r, flags=tsp.TSP_F_KV_STREAM | tsp.TSP_F_DELAY_COPY |
                           tsp.TSP_F_POISON_SLOTS).layer(xs[r], L, kv)
        torch.cuda.synchronize()
        assert torch.equal(base, streamed), f"rank {r}: K/V stream changes the result"
        assert torch.equal(base, stressed), f"rank {r}: delayed / poisoned K/V stream changes the result"
    say(f"    {cfg.fold} ranks bitwise equal")


# Several shards per launch (P = 2 at fold 8, 4 at fold 16): the QKV GEMM
# scatters each shard's Q/K/V to its own block, the attention reads each
# shard's K/V block (in place or from the slot), and the W1/W3 GEMM runs over
# the shards' W1 and W3 blocks side by side.
GROUPED = {
    # C = 128: other ranks' K/V read in place
    "fold8_inplace_d128": _cfg(hidden=1024, n_heads=8, head_dim=128, ffn=1376, seq=2048, fold=8),
    # C = 25: K/V rows copied into each shard's slot block; GQA 2, rotary, two sequences
    "fold8_ragged_gqa2_rope_b2": _cfg(hidden=512, n_heads=16, n_kv_heads=8, head_dim=32, ffn=704, seq=400,
                                      fold=8, batch=2, rope_theta=10000.0, x_std=0.02, w_std=0.045),
    # fold 16: four shards per launch, C = 20
    "fold16_c20_d32": _cfg(hidden=512, n_heads=16, head_dim=32, ffn=704, seq=640, fold=16),
}


@pytest.mark.parametrize("case", sorted(GROUPED))
def test_shards_per_launch(case):
    """Every rank's layer share with the default grouped launches and with
    one shard per launch (TSP_F_SHARD_LAUNCH), both against the oracle; the
    grouped run with delayed and NaN-poisoned slot copies bit for bit equal
    to the plain grouped run."""
    from folded_tensor_sequence_rank_amd import tsp
    cfg = GROUPED[case]
    say(f"[gpu] shards per launch {case}: h={cfg.hidden} H={cfg.n_heads} Hkv={cfg.kv_heads} d={cfg.head_dim} "
        f"S={cfg.seq} D={cfg.fold} B={cfg.batch}")
    w = synth.gen_weights(cfg)
    L = layer_dev(cfg, w)
    pos = [O.zigzag_positions(cfg.seq, cfg.fold, r) for r in range(cfg.fold)]
    xf = [synth.gen_x_rows(cfg, 0, cfg.seq, seq_index=b) for b in range(cfg.batch)]
    xs = [to_dev(np.concatenate([x[p] for x in xf]), cfg) for p in pos]
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    T = cfg.local_tokens
    for r in range(cfg.fold):
        grouped = RankRun(cfg, r).layer(xs[r], L, kv)
        single = RankRun(cfg, r, flags=tsp.TSP_F_SHARD_LAUNCH).layer(xs[r], L, kv)
        stressed = RankRun(cfg, r, flags=tsp.TSP_F_DELAY_COPY | tsp.TSP_F_POISON_SLOTS).layer(xs[r], L, kv)
        torch.cuda.synchronize()
        assert torch.equal(grouped, stressed), f"rank {r}: delayed / poisoned grouped copies change the result"
        for b in range(cfg.batch):
            ref = O.layer_rows(xf[b], w, cfg.n_heads, cfg.eps, pos[r], cfg.rope_theta)
            rows = slice(b * T, (b + 1) * T)
            _check(cfg, f"rank {r} seq {b} grouped", f64(grouped)[rows], ref)
            _check(cfg, f"rank {r} seq {b} one shard per launch", f64(single)[rows], ref)


def test_7b_s16k_rank3_full():
    """The 7B shape at 16K context, fold 8, rank 3: every output row against
    the oracle, with the other ranks' K/V read in place and, through
    TSP_F_KV_STREAM, copied into the slots on the side stream (bitwise
    equal)."""
    from folded_tensor_sequence_rank_amd import tsp
    cfg = synth.get_config("7b_s16k")
    r = cfg.ranks[0]
    say(f"[gpu] 7B shape S={cfg.seq} D={cfg.fold} rank {r}: full rank parity")
    w, x_full, L, xs, pos = _setup(cfg)
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv, skip=r)
    run = RankRun(cfg, r)
    x1 = run.attn(xs[r], L, kv)
    out = run.mlp(x1, L)
    streamed = RankRun(cfg, r, flags=tsp.TSP_F_KV_STREAM).layer(xs[r], L, kv)
    torch.cuda.synchronize()
    assert torch.equal(streamed, out), "the K/V stream changes the 16K result"
    say("    GPU done; oracle running")
    x1_ref = O.attention_block_rows(x_full, w, cfg.n_heads, cfg.eps, pos[r])
    out_ref = O.mlp_block(x1_ref, w, cfg.eps)
    xr = x_full[pos[r]].astype(np.float64)
    _check(cfg, "x1", f64(x1), x1_ref, xr, xr)
    _check(cfg, "out", f64(out), out_ref, f64(x1), x1_ref)


# Micro-batch: B independent sequences per call.  One workload per attention
# path: pipelined bf16 with the other ranks' K/V read in place, ragged bf16
# with the K/V copy, fp32, and query tiles split over key segments.
BATCH = {
    "bf16_d128_inplace_b2": SMALL["bf16_d128_inplace"].with_(batch=2),
    "bf16_d128_ragged_b3": SMALL["bf16_d128_ragged"].with_(batch=3),
    "f32_d64_b2": SMALL["f32_d64"].with_(batch=2),
    "split_b2": _cfg(hidden=512, n_heads=4, head_dim=128, ffn=1024, seq=8192, fold=2, batch=2),
}


def _batch_setup(cfg):
    """Weights, each sequence's activations (its own seeded stream), every
    rank's sequence-major local rows and the gathered K/V of all ranks."""
    B, S = cfg.batch, cfg.seq
    w = synth.gen_weights(cfg)
    L = layer_dev(cfg, w)
    xf = [synth.gen_x_rows(cfg, 0, S, seq_index=b) for b in range(B)]
    pos = [O.zigzag_positions(S, cfg.fold, r) for r in range(cfg.fold)]
    xs = [to_dev(np.concatenate([xf[b][pos[r]] for b in range(B)]), cfg) for r in range(cfg.fold)]
    return w, L, xf, pos, xs


@pytest.mark.parametrize("case", sorted(BATCH))
def test_micro_batch(case):
    """Each sequence of the batch against the oracle run on that sequence
    alone; the layer call equals the attention and MLP calls."""
    cfg = BATCH[case]
    B, T = cfg.batch, cfg.local_tokens
    say(f"[gpu] micro-batch parity {case}: B={B} S={cfg.seq} D={cfg.fold} d={cfg.head_dim} {cfg.dtype}")
    w, L, xf, pos, xs = _batch_setup(cfg)
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    for r in sorted({0, cfg.fold - 1}):
        run = RankRun(cfg, r)
        x1 = run.attn(xs[r], L, kv)
        out = run.mlp(x1, L)
        lay = run.layer(xs[r], L, kv)
        torch.cuda.synchronize()
        assert torch.equal(lay, out), "layer call differs from attention + MLP calls"
        g1, g2 = f64(x1), f64(out)
        for b in range(B):
            rows = slice(b * T, (b + 1) * T)
            x1_ref = O.attention_block_rows(xf[b], w, cfg.n_heads, cfg.eps, pos[r])
            out_ref = O.mlp_block(x1_ref, w, cfg.eps)
            xr = xf[b][pos[r]].astype(np.float64)
            _check(cfg, f"rank {r} sequence {b} x1", g1[rows], x1_ref, xr, xr)
            _check(cfg, f"rank {r} sequence {b} out", g2[rows], out_ref, g1[rows], x1_ref)


def test_7b_s16k_batch2_rank3():
    """The 7B shape at 16K context, fold 8, rank 3, two sequences per call:
    every output row of both against the oracle."""
    cfg = synth.get_config("7b_s16k").with_(batch=2)
    r, T = cfg.ranks[0], cfg.local_tokens
    say(f"[gpu] 7B shape S={cfg.seq} D={cfg.fold} B=2 rank {r}: full rank parity")
    w, L, xf, pos, xs = _batch_setup(cfg)
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv, skip=r)
    run = RankRun(cfg, r)
    x1 = run.attn(xs[r], L, kv)
    out = run.mlp(x1, L)
    torch.cuda.synchronize()
    say("    GPU done; oracle running")
    g1, g2 = f64(x1), f64(out)
    for b in range(2):
        rows = slice(b * T, (b + 1) * T)
        x1_ref = O.attention_block_rows(xf[b], w, cfg.n_heads, cfg.eps, pos[r])
        out_ref = O.mlp_block(x1_ref, w, cfg.eps)
        xr = xf[b][pos[r]].astype(np.float64)
        _check(cfg, f"sequence {b} x1", g1[rows], x1_ref, xr, xr)
        _check(cfg, f"sequence {b} out", g2[rows], out_ref, g1[rows], x1_ref)


# Rotary embedding and grouped-query attention (extensions of the layer that
# the pages do not describe).  Low-residual activations make the attention
# half dominate the output, and weights giving attention scores of std ~0.5
# (w_std^2 * h) make the rotation change that half by O(1) while keeping the
# bf16 rounding of Q and K, which grows with the scores, well inside the bar.
# Each case checks that dropping the rotation would change the output far
# beyond the bar, so a wrong angle or K/V head cannot pass.  One workload per attention
# path: fp32 (d = 16), bf16 d = 64, pipelined bf16 d = 128 reading the other
# ranks' K/V in place, ragged bf16 d = 128 with the K/V copy, and query tiles
# split over key segments with two sequences per call.
ROPE = {
    "tiny_f32_gqa2_rope": TINY.with_(fold=2, n_kv_heads=2, rope_theta=10000.0, x_std=0.02,
                                     w_std=0.2),
    "bf16_d64_gqa2_rope500": _cfg(hidden=256, n_heads=4, head_dim=64, ffn=512, seq=1024, fold=2,
                                  n_kv_heads=2, rope_theta=500.0, x_std=0.02, w_std=0.045),
    "bf16_d128_inplace_gqa4_rope": _cfg(hidden=1024, n_heads=8, ffn=1376, seq=2048, fold=4,
                                        n_kv_heads=4, rope_theta=10000.0, x_std=0.02,
                                        w_std=0.022),
    "bf16_d128_ragged_rope": _cfg(hidden=512, n_heads=4, rope_theta=10000.0, x_std=0.02,
                                  w_std=0.03),
    # one K/V head for all four query heads (multi-query attention), fold 1
    "bf16_d64_mqa_fold1_rope": _cfg(hidden=256, n_heads=4, head_dim=64, ffn=512, seq=512, fold=1,
                                    n_kv_heads=1, rope_theta=10000.0, x_std=0.02, w_std=0.045),
    "split_gqa2_rope_b2": _cfg(hidden=512, n_heads=4, head_dim=128, ffn=1024, seq=8192, fold=2,
                               batch=2, n_kv_heads=2, rope_theta=10000.0, x_std=0.02,
                               w_std=0.03),
}


@pytest.mark.parametrize("case", sorted(ROPE))
def test_rope_gqa(case):
    cfg = ROPE[case]
    B, T = cfg.batch, cfg.local_tokens
    say(f"[gpu] rotary/GQA parity {case}: H={cfg.n_heads} Hkv={cfg.kv_heads} theta={cfg.rope_theta} "
        f"B={B} S={cfg.seq} D={cfg.fold} d={cfg.head_dim} {cfg.dtype}")
    w, L, xf, pos, xs = _batch_setup(cfg)
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    for r in sorted({0, cfg.fold - 1}):
        run = RankRun(cfg, r)
        x1 = run.attn(xs[r], L, kv)
        out = run.mlp(x1, L)
        lay = run.layer(xs[r], L, kv)
        torch.cuda.synchronize()
        assert torch.equal(lay, out), "layer call differs from attention + MLP calls"
        g1, g2 = f64(x1), f64(out)
        for b in range(B):
            rows = slice(b * T, (b + 1) * T)
            x1_ref = O.attention_block_rows(xf[b], w, cfg.n_heads, cfg.eps, pos[r], cfg.rope_theta)
            out_ref = O.mlp_block(x1_ref, w, cfg.eps)
            xr = xf[b][pos[r]].astype(np.float64)
            _check(cfg, f"rank {r} sequence {b} x1", g1[rows], x1_ref, xr, xr)
            _check(cfg, f"rank {r} sequence {b} out", g2[rows], out_ref, g1[rows], x1_ref)
            plain = O.attention_block_rows(xf[b], w, cfg.n_heads, cfg.eps, pos[r], 0.0)
            seen = rel_fro(g1[rows] - xr, plain - xr)
            say(f"    without the rotation the attention delta would differ by {seen:.2e}")
            assert seen > 10 * tol(cfg), "the rotation barely changes this case"


def test_7b_s16k_gqa8_rope_rank3():
    """The 7B shape at 16K context, fold 8, rank 3, with the rotary embedding
    (base 10^4) and 8 K/V heads (one per rank): every output row against the
    oracle."""
    cfg = synth.get_config("7b_s16k").with_(n_kv_heads=8, rope_theta=10000.0)
    r = cfg.ranks[0]
    say(f"[gpu] 7B shape S={cfg.seq} D={cfg.fold} Hkv=8 rotary rank {r}: full rank parity")
    w, x_full, L, xs, pos = _setup(cfg)
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv, skip=r)
    run = RankRun(cfg, r)
    x1 = run.attn(xs[r], L, kv)
    out = run.mlp(x1, L)
    torch.cuda.synchronize()
    say("    GPU done; oracle running")
    x1_ref = O.attention_block_rows(x_full, w, cfg.n_heads, cfg.eps, pos[r], cfg.rope_theta)
    out_ref = O.mlp_block(x1_ref, w, cfg.eps)
    xr = x_full[pos[r]].astype(np.float64)
    _check(cfg, "x1", f64(x1), x1_ref, xr, xr)
    _check(cfg, "out", f64(out), out_ref, f64(x1), x1_ref)


# Degenerate zigzags: one and two tokens per chunk (S = 2D, 4D), so every
# GEMM, attention tile and K/V copy is almost all ragged tail; with three
# sequences, grouped K/V and the rotary embedding on, and with 128-dim heads
# (the pipelined kernel's shape, here on the copied-K/V path since C % 64 != 0).
EDGE = {
    "c1_fold8_b3_gqa2_rope": _cfg(hidden=256, n_heads=16, head_dim=16, ffn=176, seq=16, fold=8,
                                  batch=3, n_kv_heads=8, rope_theta=10000.0),
    "c2_fold4_gqa2_rope_f32": _cfg(hidden=128, n_heads=8, head_dim=16, ffn=176, seq=16, fold=4,
                                   n_kv_heads=4, rope_theta=100.0, dtype="f32"),
    "c1_fold4_d128_b2": _cfg(hidden=512, n_heads=4, head_dim=128, ffn=688, seq=8, fold=4, batch=2),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_degenerate_chunks(case):
    cfg = EDGE[case]
    B, T = cfg.batch, cfg.local_tokens
    say(f"[gpu] degenerate zigzag {case}: C={cfg.chunk} S={cfg.seq} D={cfg.fold} B={B} "
        f"Hkv={cfg.kv_heads} theta={cfg.rope_theta} d={cfg.head_dim} {cfg.dtype}")
    w, L, xf, pos, xs = _batch_setup(cfg)
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    for r in range(cfg.fold):
        run = RankRun(cfg, r)
        out = run.layer(xs[r], L, kv)
        torch.cuda.synchronize()
        g = f64(out)
        for b in range(B):
            ref = O.rank_share(xf[b], w, cfg.n_heads, cfg.eps, cfg.seq, cfg.fold, r, cfg.rope_theta)
            _check(cfg, f"rank {r} sequence {b} out", g[b * T:(b + 1) * T], ref)


def test_rope_largest_positions_f32():
    """The rotary embedding at positions up to 131071 (rank 0 of 8 holds the
    last zigzag chunk), in fp32.  The rotated K rows that tsp_kv_shard writes
    into the gathered K/V are compared element by element with the oracle's:
    angles formed in single precision would be off by ~1e-3 rad here and
    move K by ~7e-4 (relative), far beyond the 2e-5 bar.  Sampled rows of the
    attention half are checked at the fp32 bar as well."""
    cfg = _cfg(hidden=256, n_heads=8, head_dim=32, ffn=512, seq=131072, fold=8, dtype="f32",
               rope_theta=10000.0, x_std=0.02, w_std=0.06)
    r, d, S = 0, cfg.head_dim, cfg.seq
    say(f"[gpu] rotary embedding at positions up to {S - 1}, fp32, rank {r}")
    w, x_full, L, xs, pos = _setup(cfg)
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    x1 = RankRun(cfg, r).attn(xs[r], L, kv)
    torch.cuda.synchronize()
    C = cfg.chunk
    local = np.r_[0:8, C - 8:C, C:C + 8, 2 * C - 24:2 * C]   # chunk edges; the last rows end at S - 1
    p = pos[r][local]
    assert p.max() == S - 1
    # K and V of every head at these positions: block j holds head j (one per shard)
    kvh = f64(kv).reshape(cfg.fold, 2, S, d)  # [shard][K | V^T][...]
    n1 = O.rmsnorm(x_full[p], w.g1, cfg.eps)
    worst = 0.0
    for j in range(cfg.fold):
        c = slice(j * d, (j + 1) * d)
        k_ref = O.rope(n1 @ np.asarray(w.wk[:, c], np.float64), p, cfg.rope_theta)
        v_ref = n1 @ np.asarray(w.wv[:, c], np.float64)
        k_gpu = kvh[j, 0][p]
        v_gpu = kvh[j, 1].reshape(d, S)[:, p].T
        ek, ev = rel_fro(k_gpu, k_ref), rel_fro(v_gpu, v_ref)
        assert ek < 2e-5 and ev < 2e-5, (j, ek, ev)
        worst = max(worst, ek)
    say(f"    rotated K of all heads at positions {p.min()}..{p.max()}: rel error {worst:.2e} (bar 2e-5)")
    ref = O.attention_block_rows(x_full, w, cfg.n_heads, cfg.eps, p, cfg.rope_theta)
    xr = x_full[p].astype(np.float64)
    _check(cfg, "x1 (sampled rows)", f64(x1)[local], ref, xr, xr)
