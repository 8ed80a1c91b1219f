"""Device-side set-up for the GPU parity tests and the benchmark.

Builds one layer's device inputs from the seeded generator, produces the
other ranks' K/V rows with tsp_kv_shard (the all-gather's payload), and runs
a rank's share through the C ABI.  The gathered K/V buffer starts as NaN, so
any read of a row the rank never receives (its own rows, or rows past its
causal window) shows up in the output.
"""
import sys
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

import synth
from folded_tensor_sequence_rank_amd import tsp

DEV = "cuda"


def tdtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, cfg) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(tdtype(cfg))


@dataclass
class LayerDev:
    g1: torch.Tensor
    g2: torch.Tensor
    w_attn: List[torch.Tensor]
    w_mlp: List[torch.Tensor]


def layer_dev(cfg, w) -> LayerDev:
    D = cfg.fold
    return LayerDev(
        g1=to_dev(w.g1, cfg), g2=to_dev(w.g2, cfg),
        w_attn=tsp.pack_attn_shards(*(to_dev(m, cfg) for m in (w.wq, w.wk, w.wv, w.wo)), D),
        w_mlp=tsp.pack_mlp_shards(*(to_dev(m, cfg) for m in (w.w1, w.w3, w.w2)), D))


def local_rows(cfg, x_full_rows_fn, r) -> np.ndarray:
    """Rank r's local rows, gathered with the library's own zigzag helper."""
    pos = tsp.zigzag_positions(cfg.seq, cfg.fold, r)
    return x_full_rows_fn(pos)


def new_kv(cfg) -> torch.Tensor:
    return torch.full((tsp.kv_elems(cfg),), float("nan"), dtype=tdtype(cfg), device=DEV)


def ws_for(cfg, r, which, flags=0) -> torch.Tensor:
    n = tsp.workspace_bytes(tsp.make_dims(cfg, r, flags), which)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=DEV)


def fill_kv(cfg, L: LayerDev, xs_dev: List[torch.Tensor], kv: torch.Tensor, skip: Optional[int] = None):
    """tsp_kv_shard for every rank (except `skip`): the gathered K/V."""
    ws = ws_for(cfg, 0, tsp.TSP_WS_KV)
    for r in range(cfg.fold):
        if r == skip:
            continue
        tsp.tsp_kv_shard(tsp.make_dims(cfg, r), xs_dev[r], L.g1, L.w_attn, kv, ws)


class RankRun:
    """Runs rank r's attention half, MLP half and whole layer."""

    def __init__(self, cfg, r, flags=0, copy_stream=True):
        self.cfg, self.r = cfg, r
        self.dims = tsp.make_dims(cfg, r, flags)
        self.ws_a = ws_for(cfg, r, tsp.TSP_WS_ATTN, flags)
        self.ws_m = ws_for(cfg, r, tsp.TSP_WS_MLP, flags)
        self.ws_l = ws_for(cfg, r, tsp.TSP_WS_LAYER, flags)
        self.cs = torch.cuda.Stream() if copy_stream else None

    def attn(self, x, L: LayerDev, kv):
        x1 = torch.empty_like(x)
        tsp.tsp_attn_shard(self.dims, x, L.g1, L.w_attn, kv, x1, self.ws_a, copy_stream=self.cs)
        return x1

    def attn_save(self, x, L: LayerDev, kv):
        """tsp_attn_shard_save: x1, the attention output A [B*T][h] and the
        rows' log2 softmax normalisers [H][B*T]."""
        cfg = self.cfg
        x1, a = torch.empty_like(x), torch.empty_like(x)
        lse = torch.empty(cfg.n_heads * x.shape[0], dtype=torch.float32, device=DEV)
        tsp.tsp_attn_shard_save(self.dims, x, L.g1, L.w_attn, kv, x1, a, lse, self.ws_a, copy_stream=self.cs)
        return x1, a, lse

    def mlp(self, x1, L: LayerDev):
        out = torch.empty_like(x1)
        tsp.tsp_mlp_shard(self.dims, x1, L.g2, L.w_mlp, out, self.ws_m, copy_stream=self.cs)
        return out

    def layer(self, x, L: LayerDev, kv, out=None):
        out = torch.empty_like(x) if out is None else out
        tsp.tsp_layer_shard(self.dims, x, L.g1, L.w_attn, kv, L.g2, L.w_mlp, out, self.ws_l,
                            copy_stream=self.cs)
        return out


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


from parity import rel_fro, tol  # noqa: E402,F401  (the parity bar lives in tests/parity.py)
