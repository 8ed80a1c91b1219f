"""The layer call under HIP graph capture: the library's path (kernels,
side-stream copies and the events that order them) is capturable; every
replay, with eager work between replays, is bitwise equal to the eager call."""
import numpy as np
import pytest
import torch

import synth
from folded_tensor_sequence_rank_amd import tsp
from gpu_harness import RankRun, fill_kv, layer_dev, new_kv, say, to_dev

pytestmark = pytest.mark.gpu


def _cfg(**kw):
    base = dict(name="case", hidden=512, n_heads=4, head_dim=128, ffn=1376, seq=2048, fold=4,
                ranks=(1,), layers=1, dtype="bf16")
    base.update(kw)
    return synth.LayerConfig(**base)


CASES = {
    "bf16_d128_inplace": _cfg(),
    "split_gqa2_rope_b2": _cfg(ffn=1024, seq=8192, fold=2, batch=2, n_kv_heads=2, rope_theta=1e4),
    "f32_ragged": _cfg(hidden=256, n_heads=4, head_dim=64, ffn=688, seq=1600, dtype="f32"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_layer_graph_replay_bitwise(case):
    cfg = CASES[case]
    r = cfg.ranks[0]
    say(f"[gpu] graph capture of tsp_layer_shard: {case}")
    L = layer_dev(cfg, synth.gen_weights(cfg))
    xs = [to_dev(np.concatenate([synth.gen_rows(cfg, tsp.zigzag_positions(cfg.seq, cfg.fold, q),
                                                seq_index=b) for b in range(cfg.batch)]), cfg)
          for q in range(cfg.fold)]
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv, skip=r)
    run = RankRun(cfg, r)
    x, out = xs[r], torch.empty_like(xs[r])
    run.layer(x, L, kv, out)
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    out.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run.layer(x, L, kv, out)
    torch.cuda.synchronize()
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager call"
        run.layer(x, L, kv, out)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    say("    3 replays bitwise equal to the eager call")
