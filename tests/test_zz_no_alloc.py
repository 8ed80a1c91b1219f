"""tsp_layer_shard_noalloc (the static-scratch variant of tsp_layer_shard)
against tsp_layer_shard, through the C ABI: bit-for-bit equal outputs on two
calls in a row, the second with a smaller input, so the second runs on
scratch that still holds the first call's (larger) contents; and a shape
past the scratch is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import synth
from folded_tensor_sequence_rank_amd import tsp
from gpu_harness import RankRun, fill_kv, layer_dev, new_kv, say, to_dev

pytestmark = pytest.mark.gpu


def _case(cfg, r):
    w = synth.gen_weights(cfg)
    L = layer_dev(cfg, w)
    pos = [tsp.zigzag_positions(cfg.seq, cfg.fold, q) for q in range(cfg.fold)]
    xs = [to_dev(np.concatenate([synth.gen_rows(cfg, p, seq_index=b) for b in range(cfg.batch)]), cfg)
          for p in pos]
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv, skip=r)
    return L, xs[r], kv


def test_noalloc_matches_layer_shard_on_two_calls():
    # one shard per launch: 241 MiB of the 256 MiB scratch (the default
    # launch grouping would need 495 MiB at this size)
    big = synth.get_config("7b_s16k").with_(seq=4096)
    small = synth.LayerConfig(name="small", hidden=512, n_heads=4, head_dim=128, ffn=688, seq=1600,
                              fold=2, batch=2, n_kv_heads=2, rope_theta=10000.0)
    cs = torch.cuda.Stream()
    for cfg, r, flags in ((big, 3, tsp.TSP_F_SHARD_LAUNCH), (small, 1, 0)):
        d = tsp.make_dims(cfg, r, flags)
        need = tsp.workspace_bytes(d, tsp.TSP_WS_LAYER)
        assert 0 < need <= tsp.NOALLOC_SCRATCH_BYTES
        say(f"[gpu] no-alloc layer: h={cfg.hidden} S={cfg.seq} D={cfg.fold} B={cfg.batch} rank {r} "
            f"flags {flags}, {need / 2**20:.1f} MiB of scratch")
        L, x, kv = _case(cfg, r)
        ref = RankRun(cfg, r, flags).layer(x, L, kv)
        out = torch.full_like(x, float("nan"))
        tsp.tsp_layer_shard_noalloc(d, x, L.g1, L.w_attn, kv, L.g2, L.w_mlp, out, copy_stream=cs)
        again = torch.full_like(x, float("nan"))
        tsp.tsp_layer_shard_noalloc(d, x, L.g1, L.w_attn, kv, L.g2, L.w_mlp, again)  # no side stream
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        assert torch.equal(out, ref), "no-alloc output differs from tsp_layer_shard"
        assert torch.equal(again, ref), "no-alloc output without a copy stream differs"
        del L, x, kv


def test_noalloc_refuses_shapes_past_the_scratch():
    cfg = synth.get_config("7b_s16k")                            # over 400 MiB
    d = tsp.make_dims(cfg, 3)
    assert tsp.workspace_bytes(d, tsp.TSP_WS_LAYER) > tsp.NOALLOC_SCRATCH_BYTES
    x = torch.empty(cfg.local_tokens * cfg.hidden, dtype=torch.bfloat16, device="cuda")
    g = torch.empty(cfg.hidden, dtype=torch.bfloat16, device="cuda")
    wa = [torch.empty(16, dtype=torch.bfloat16, device="cuda")] * cfg.fold
    with pytest.raises(tsp.TspError) as e:  # plain pointers: nothing is enqueued
        tsp._check(tsp.lib().tsp_layer_shard_noalloc(
            tsp.ctypes.byref(d), x.data_ptr(), g.data_ptr(), tsp._ptrs(wa), x.data_ptr(), g.data_ptr(),
            tsp._ptrs(wa), x.data_ptr(), None, None))
    assert e.value.name == "TSP_E_WORKSPACE" and "static scratch" in str(e.value)
