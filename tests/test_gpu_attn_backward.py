"""GPU parity of the attention core's backward (tsp_attn_core_backward)
against the backward oracle, head by head: dQ of the rank's rows, and the
rank's partial dK / dV of every position (summed over the query heads that
share a K/V head).  Inputs are seeded standard normals, so the scores
q.k / sqrt(d) have unit spread and the softmax is far from uniform."""
import numpy as np
import pytest
import torch

import oracle.tsp_oracle as O
import oracle.tsp_oracle_bwd as B
import synth
from folded_tensor_sequence_rank_amd import tsp
from gpu_harness import DEV, f64, rel_fro, say

pytestmark = pytest.mark.gpu

TOL = 1e-2  # relative Frobenius, bf16 operands


def _cfg(**kw):
    base = dict(name="case", hidden=512, n_heads=4, head_dim=128, ffn=1024, seq=2048, fold=2,
                ranks=(1,), layers=1, dtype="bf16")
    base.update(kw)
    return synth.LayerConfig(**base)


CASES = {
    # several 64-row tiles per chunk, both chunks' key ranges
    "d128_fold2_rank1": (_cfg(), 1),
    "d128_fold4_rank0": (_cfg(fold=4), 0),
    "d128_fold4_rank3": (_cfg(fold=4), 3),
    # ragged chunks (C = 200, not a multiple of 64), two sequences, d = 64
    "d64_ragged_b2": (_cfg(hidden=256, head_dim=64, seq=1600, fold=4, batch=2), 2),
    # grouped K/V heads: 4 query heads on one K/V head per shard
    "gqa4_d128": (_cfg(hidden=1024, n_heads=8, n_kv_heads=2, seq=1024), 1),
    # the 7B head group (4 heads of 128) at S = 16384, fold 8, rank 3
    "7b_group_s16k_rank3": (_cfg(hidden=4096, n_heads=32, head_dim=128, ffn=11008, seq=16384, fold=8), 3),
}


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("case", sorted(CASES))
def test_attention_core_backward(case):
    cfg, r = CASES[case]
    D, d, S = cfg.fold, cfg.head_dim, cfg.seq
    Bn = cfg.batch
    T = S // D
    Hd, Hkd = cfg.n_heads // D, cfg.kv_heads // D
    grp = Hd // Hkd
    say(f"[gpu] attention backward {case}: d={d} S={S} D={D} B={Bn} Hd={Hd} Hkd={Hkd} rank {r}")
    rng = np.random.default_rng(1234 + r)
    q = _bf16(rng.standard_normal((Hd, Bn * T, d)))
    k = _bf16(rng.standard_normal((Hkd, Bn * S, d)))
    v = _bf16(rng.standard_normal((Hkd, Bn * S, d)))
    do = _bf16(rng.standard_normal((Bn * T, Hd * d)))
    kv = torch.cat([k.reshape(-1), v.transpose(1, 2).contiguous().reshape(-1)]).to(DEV)
    dims = tsp.make_dims(cfg, r)
    ws = torch.empty(max(tsp.workspace_bytes(dims, tsp.TSP_WS_ATTN_BWD), 256), dtype=torch.uint8, device=DEV)
    dq = torch.full((Hd, Bn * T, d), float("nan"), device=DEV)
    dk = torch.full((Hkd, Bn * S, d), float("nan"), device=DEV)
    dv = torch.full((Hkd, Bn * S, d), float("nan"), device=DEV)
    tsp.tsp_attn_core_backward(dims, q.to(DEV), kv, do.to(DEV), dq, dk, dv, ws)
    torch.cuda.synchronize()
    say("    GPU done; oracle running")
    qn, kn, vn, don = f64(q), f64(k), f64(v), f64(do)
    dq_g, dk_g, dv_g = f64(dq), f64(dk), f64(dv)
    pos = O.zigzag_positions(S, D, r)
    for b in range(Bn):
        rows, keys = slice(b * T, (b + 1) * T), slice(b * S, (b + 1) * S)
        for hk in range(Hkd):
            gk = np.zeros((S, d))
            gv = np.zeros((S, d))
            for t in range(hk * grp, (hk + 1) * grp):
                eq, ek, ev = B.causal_attention_backward(qn[t, rows], pos, kn[hk, keys], vn[hk, keys],
                                                         don[rows, t * d:(t + 1) * d])
                e = rel_fro(dq_g[t, rows], eq)
                say(f"    seq {b} head {t} dQ: rel {e:.3e}")
                assert e <= TOL, (b, t, e)
                gk += ek
                gv += ev
            for name, got, want in (("dK", dk_g[hk, keys], gk), ("dV", dv_g[hk, keys], gv)):
                e = rel_fro(got, want)
                say(f"    seq {b} K/V head {hk} {name}: rel {e:.3e}")
                assert e <= TOL, (b, hk, name, e)
                # no query of the rank reaches past its last position
                assert np.all(got[pos.max() + 1:] == 0.0), name


def test_attention_core_backward_7b_s64k_rank3():
    """The shape and launch the attention-backward benchmark times (7B head
    group, S = 65536, fold 8, rank 3): dQ on 96 sampled rows of every head
    (a row's dQ depends on that row alone), and dK, dV of K/V head 0 at every
    position, the oracle summing all 8192 query rows in chunks."""
    cfg = _cfg(hidden=4096, n_heads=32, head_dim=128, ffn=11008, seq=65536, fold=8)
    r, D, d, S = 3, 8, 128, 65536
    T, Hd = S // D, 4
    say(f"[gpu] attention backward 7B group S={S} D={D} rank {r}")
    rng = np.random.default_rng(4321)
    q = _bf16(rng.standard_normal((Hd, T, d)))
    k = _bf16(rng.standard_normal((Hd, S, d)))
    v = _bf16(rng.standard_normal((Hd, S, d)))
    do = _bf16(rng.standard_normal((T, Hd * d)))
    kv = torch.cat([k.reshape(-1), v.transpose(1, 2).contiguous().reshape(-1)]).to(DEV)
    dims = tsp.make_dims(cfg, r)
    ws = torch.empty(tsp.workspace_bytes(dims, tsp.TSP_WS_ATTN_BWD), dtype=torch.uint8, device=DEV)
    dq = torch.full((Hd, T, d), float("nan"), device=DEV)
    dk = torch.full((Hd, S, d), float("nan"), device=DEV)
    dv = torch.full((Hd, S, d), float("nan"), device=DEV)
    tsp.tsp_attn_core_backward(dims, q.to(DEV), kv, do.to(DEV), dq, dk, dv, ws)
    torch.cuda.synchronize()
    say("    GPU done; oracle running")
    qn, kn, vn, don = f64(q), f64(k), f64(v), f64(do)
    pos = O.zigzag_positions(S, D, r)
    # both chunks' edges and interior rows
    rows = np.unique(np.concatenate([[0, 1, T // 2 - 1, T // 2, T - 1], rng.integers(0, T, 91)]))
    for t in range(Hd):
        eq, _, _ = B.causal_attention_backward(qn[t, rows], pos[rows], kn[t], vn[t], don[rows, t * d:(t + 1) * d])
        e = rel_fro(f64(dq[t, rows]), eq)
        say(f"    head {t} dQ on {rows.size} rows: rel {e:.3e}")
        assert e <= TOL, (t, e)
    gk = np.zeros((S, d))
    gv = np.zeros((S, d))
    for c0 in range(0, T, 1024):
        c = slice(c0, c0 + 1024)
        _, ek, ev = B.causal_attention_backward(qn[0, c], pos[c], kn[0], vn[0], don[c, :d])
        gk += ek
        gv += ev
    for name, got, want in (("dK", f64(dk[0]), gk), ("dV", f64(dv[0]), gv)):
        e = rel_fro(got, want)
        say(f"    K/V head 0 {name}: rel {e:.3e}")
        assert e <= TOL, (name, e)
        assert np.all(got[pos.max() + 1:] == 0.0), name
