"""The parity bar itself (tests/parity.py), checked on the CPU against
planted localized errors in oracle results: the local (row, head-sized
block) bound must catch one head of one query tile off by 20%, which the
whole-tensor bound alone lets through, and must pass the oracle's exact
values as a bf16 output would store them."""
import numpy as np
import pytest

import oracle.tsp_oracle as O
import synth
from parity import compare, storage_round

# low-residual activations, 32 heads: the attention delta dominates x1
CFG = synth.LayerConfig(name="local", hidden=512, n_heads=32, head_dim=16, ffn=1024, seq=4096,
                        fold=1, dtype="bf16", x_std=0.02)


@pytest.fixture(scope="module")
def attn_case():
    cfg = CFG
    w = synth.gen_weights(cfg)
    x = synth.gen_x_rows(cfg, 0, cfg.seq).astype(np.float64)
    rows = np.arange(cfg.seq)
    n1 = O.rmsnorm(x, w.g1, cfg.eps)
    a = O.multihead_causal(n1, rows, w, cfg.n_heads, 0.0)
    x1 = x + a @ np.asarray(w.wo, np.float64)
    return cfg, w, x, a, x1


def _plant(cfg, w, a, x1, head, tile, factor):
    """x1 with head `head`'s attention output of query rows
    [128*tile, 128*tile + 128) scaled by `factor`."""
    d = cfg.head_dim
    c = slice(head * d, (head + 1) * d)
    r = slice(128 * tile, 128 * tile + 128)
    out = x1.copy()
    out[r] += (factor - 1.0) * a[r, c] @ np.asarray(w.wo, np.float64)[c, :]
    return out


def test_exact_values_stored_in_bf16_pass(attn_case):
    cfg, w, x, a, x1 = attn_case
    ok, msg, st = compare(cfg, storage_round(cfg, x1), x1, x, x)
    assert ok, msg


@pytest.mark.parametrize("head,tile", [(3, 12), (7, 5), (31, 31)])
def test_one_head_of_one_tile_off_by_20_percent_is_caught(attn_case, head, tile):
    cfg, w, x, a, x1 = attn_case
    bad = storage_round(cfg, _plant(cfg, w, a, x1, head, tile, 1.2))
    ok, msg, st = compare(cfg, bad, x1, x, x)
    assert not ok, msg
    assert not st["delta_block_ok"]
    # the whole-tensor bounds alone would have passed it
    assert st["rel"] <= 1e-2 and st["delta_rel"] <= 1e-2 + 1.25 * 3e-3, st


def test_one_split_segment_dropped_is_caught(attn_case):
    """A merge that loses one key segment of one query tile (every head of
    its rows attends to a subset of its keys)."""
    cfg, w, x, a, x1 = attn_case
    r = slice(3968, 4096)                        # the last query tile: keys 0..4095
    rows = np.arange(3968, 4096)
    n1 = O.rmsnorm(x, w.g1, cfg.eps)
    d = cfg.head_dim
    a_bad = a.copy()
    for t in range(cfg.n_heads):
        c = slice(t * d, (t + 1) * d)
        q = n1[rows] @ np.asarray(w.wq[:, c], np.float64)
        k = n1 @ np.asarray(w.wk[:, c], np.float64)
        v = n1 @ np.asarray(w.wv[:, c], np.float64)
        # keys [1024, 2048) missing from the merge
        keep = np.r_[0:1024, 2048:4096]
        a_bad[r, c] = O.causal_attention(q, rows - 1024, k[keep], v[keep])
    bad = storage_round(cfg, x + a_bad @ np.asarray(w.wo, np.float64))
    ok, msg, st = compare(cfg, bad, x1, x, x)
    assert not ok and not st["delta_block_ok"], msg


def test_error_spread_evenly_passes(attn_case):
    """A correct kernel's rounding noise: every attention output element off
    by an independent 0.5% (about the measured bf16 error) passes."""
    cfg, w, x, a, x1 = attn_case
    rng = np.random.default_rng(1)
    noisy = a * (1.0 + 5e-3 * rng.standard_normal(a.shape))
    got = storage_round(cfg, x + noisy @ np.asarray(w.wo, np.float64))
    ok, msg, st = compare(cfg, got, x1, x, x)
    assert ok, msg
