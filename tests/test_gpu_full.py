"""GPU parity at the full workload sizes, on sampled rows.

The expected rows were written by tests/golden/make_golden.py, which calls
only the CPU oracle on the seeded generator's inputs.  The HIP path runs the
real shapes through the C ABI (every rank's K/V produced by tsp_kv_shard, the
rank's own rows in the gathered buffer left as NaN), and its outputs at the
stored local rows must match the bar of tests/parity.py on the sampled rows:
relative Frobenius error <= 1e-2, the block deltas within the rounding-aware
bound, and every (row, 128-column block) within twice that.
"""
import hashlib
import os

import numpy as np
import pytest
import torch

import synth
from folded_tensor_sequence_rank_amd import tsp
from gpu_harness import RankRun, f64, fill_kv, layer_dev, new_kv, say, to_dev
from test_gpu_parity import _check

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _source_hash():
    h = hashlib.sha256()
    for f in ("synth/gen.py", "synth/configs.py", "oracle/tsp_oracle.py"):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def _golden(name):
    path = os.path.join(GOLDEN, f"{name}.npz")
    if not os.path.exists(path):
        pytest.fail(f"{path} missing: run tests/golden/make_golden.py {name}")
    g = np.load(path, allow_pickle=False)
    if str(g["source_sha256_16"]) != _source_hash():
        pytest.fail(f"{path} was made from other generator/oracle sources: regenerate it")
    return g


def _inputs(cfg, layer=0):
    w = synth.gen_weights(cfg, layer)
    L = layer_dev(cfg, w)
    del w
    return L


@pytest.mark.parametrize("name", ["7b_s64k", "7b_s64k_lowres", "7b_s128k", "7b_rope_s64k",
                                  "7b_gqa8_rope_s64k", "7b_s16k_b4"])
def test_full_size_single_layer(name):
    """Sampled rows -- chunk edges and one row of every 128-row query tile of
    each rank (and sequence) -- against the oracle, at the workload's full
    shape and launch configuration."""
    cfg = synth.get_config(name)
    g = _golden(name)
    B, T = cfg.batch, cfg.local_tokens
    say(f"[gpu] full-size parity {name}: S={cfg.seq} D={cfg.fold} B={B} ranks {cfg.ranks}")
    L = _inputs(cfg)
    pos = [tsp.zigzag_positions(cfg.seq, cfg.fold, r) for r in range(cfg.fold)]
    xs_host = [np.concatenate([synth.gen_rows(cfg, p, seq_index=b) for b in range(B)]) for p in pos]
    xs = [to_dev(x, cfg) for x in xs_host]
    times = {}
    for r in cfg.ranks:
        kv = new_kv(cfg)
        fill_kv(cfg, L, xs, kv, skip=r)
        run = RankRun(cfg, r)
        x1 = run.attn(xs[r], L, kv)
        out = run.mlp(x1, L)
        lay = run.layer(xs[r], L, kv)
        # attention time of this rank (zigzag balance), median of 3
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(3)]
        for e0, e1 in ev:
            e0.record()
            run.attn(xs[r], L, kv)
            e1.record()
        torch.cuda.synchronize()
        times[r] = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[1]
        x1_all, out_all = f64(x1), f64(out)
        for b in range(B):
            key = f"r{r}" if B == 1 else f"r{r}_s{b}"
            local = g[f"{key}_local"]
            assert np.array_equal(pos[r][local], g[f"{key}_pos"])
            rows = b * T + local
            xr = xs_host[r][rows].astype(np.float64)
            gx1 = g[f"{key}_x1"].astype(np.float64)
            gout = g[f"{key}_out"].astype(np.float64)
            x1s = x1_all[rows]
            tag = f"rank {r}" + ("" if B == 1 else f" sequence {b}")
            _check(cfg, f"{tag} x1 ({len(local)} sampled rows)", x1s, gx1, xr, xr)
            _check(cfg, f"{tag} out ({len(local)} sampled rows)", out_all[rows], gout, x1s, gx1)
        assert torch.equal(lay, out), "layer call differs from attention + MLP calls"
        assert torch.isfinite(out).all()
        say(f"    rank {r}: attention half {times[r]:.2f} ms")
        del kv
    if len(times) > 1:  # equal causal work per rank -> similar time
        t = list(times.values())
        assert max(t) / min(t) < 1.3, f"zigzag ranks differ in time: {times}"


def test_full_fold_four_layers():
    """All 4 ranks of a 4-layer stack at S=32768, fold 4, run one after
    another layer by layer; sampled rows of the final output."""
    name = "7b_fold4_s32k_4layer"
    cfg = synth.get_config(name)
    g = _golden(name)
    say(f"[gpu] full fold {name}: {cfg.layers} layers x {cfg.fold} ranks, S={cfg.seq}")
    pos = [tsp.zigzag_positions(cfg.seq, cfg.fold, r) for r in range(cfg.fold)]
    xs = [to_dev(synth.gen_rows(cfg, p, 0), cfg) for p in pos]
    for layer in range(cfg.layers):
        L = _inputs(cfg, layer)
        kv = new_kv(cfg)
        fill_kv(cfg, L, xs, kv)
        xs = [RankRun(cfg, r).layer(xs[r], L, kv) for r in range(cfg.fold)]
        torch.cuda.synchronize()
        say(f"    layer {layer} done")
        del kv, L
    for r in range(cfg.fold):
        local = g[f"r{r}_local"]
        assert np.array_equal(pos[r][local], g[f"r{r}_pos"])
        _check(cfg, f"rank {r} out after {cfg.layers} layers (sampled)", f64(xs[r])[local],
               g[f"r{r}_out"].astype(np.float64))
