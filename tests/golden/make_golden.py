"""Writes the sampled expected outputs of the full-size workloads.

Calls only the CPU oracle (oracle/tsp_oracle.py) on the seeded generator's
inputs (synth/).  For each workload, rank (and sequence of a micro-batch) it
picks local rows -- first, middle and last of each zigzag chunk, and one
seeded random row in every 128-row query tile, so that every attention work
item's rows are represented -- and stores the oracle's layer output there
and, for one-layer workloads, the attention half x1 as well.  The GPU tests compare the HIP path with these
rows.  Each file records the sha256 of the generator and oracle sources it
was made from, so a change to either is detected.

Usage: python tests/golden/make_golden.py [workload ...]
"""
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle.tsp_oracle as O  # noqa: E402
import synth  # noqa: E402

WORKLOADS = ["7b_s64k", "7b_s64k_lowres", "7b_s128k", "7b_fold4_s32k_4layer", "7b_rope_s64k",
             "7b_gqa8_rope_s64k", "7b_s16k_b4"]
TILE = 128  # local query rows per attention work item


def source_hash():
    h = hashlib.sha256()
    for f in ("synth/gen.py", "synth/configs.py", "oracle/tsp_oracle.py"):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def sample_rows(cfg, r, b=0):
    """Chunk edges and one seeded row in each 128-row query tile of rank r
    (sequence b of a micro-batch)."""
    C, T = cfg.chunk, cfg.local_tokens
    local = [0, C // 2, C - 1, C, C + C // 2, 2 * C - 1]
    rng = np.random.default_rng([cfg.seed, r, 7, b])
    for t0 in range(0, T, TILE):
        local.append(t0 + int(rng.integers(0, min(TILE, T - t0))))
    local = sorted(set(local))
    pos = O.zigzag_positions(cfg.seq, cfg.fold, r)[local]
    return np.array(local, np.int64), pos


def main(names):
    for name in names:
        cfg = synth.get_config(name)
        t0 = time.time()
        out = {"workload": name, "source_sha256_16": source_hash()}
        rows = {r: sample_rows(cfg, r) for r in cfg.ranks}
        pmax = int(max(p.max() for _, p in rows.values())) + 1
        if cfg.batch > 1:
            # every sequence of the micro-batch: its own activations, its own rows
            w = synth.gen_weights(cfg)
            for b in range(cfg.batch):
                x = synth.gen_x_rows(cfg, 0, cfg.seq, seq_index=b)
                for r in cfg.ranks:
                    local, pos = sample_rows(cfg, r, b)
                    x1 = O.attention_block_rows(x, w, cfg.n_heads, cfg.eps, pos, cfg.rope_theta)
                    y = O.mlp_block(x1, w, cfg.eps)
                    out[f"r{r}_s{b}_local"] = local
                    out[f"r{r}_s{b}_pos"] = pos
                    out[f"r{r}_s{b}_x1"] = x1.astype(np.float32)
                    out[f"r{r}_s{b}_out"] = y.astype(np.float32)
                    print(f"{name} rank {r} sequence {b}: {len(pos)} rows, {time.time() - t0:.0f}s",
                          flush=True)
        elif cfg.layers == 1:
            x = synth.gen_x_rows(cfg, 0, pmax)
            w = synth.gen_weights(cfg)
            for r, (local, pos) in rows.items():
                x1 = O.attention_block_rows(x, w, cfg.n_heads, cfg.eps, pos, cfg.rope_theta)
                y = O.mlp_block(x1, w, cfg.eps)
                out[f"r{r}_local"] = local
                out[f"r{r}_pos"] = pos
                out[f"r{r}_x1"] = x1.astype(np.float32)
                out[f"r{r}_out"] = y.astype(np.float32)
                print(f"{name} rank {r}: {len(pos)} rows, {time.time() - t0:.0f}s", flush=True)
        else:
            # every layer's input comes from the generator's layer-0 activations
            x = synth.gen_x_rows(cfg, 0, cfg.seq)
            ws = [synth.gen_weights(cfg, l) for l in range(cfg.layers)]
            allpos = np.concatenate([p for _, p in rows.values()])
            y = O.stack_rows(x, ws, cfg.n_heads, cfg.eps, allpos, cfg.rope_theta)
            k = 0
            for r, (local, pos) in rows.items():
                out[f"r{r}_local"] = local
                out[f"r{r}_pos"] = pos
                out[f"r{r}_out"] = y[k:k + len(pos)].astype(np.float32)
                k += len(pos)
            print(f"{name}: {len(allpos)} rows over {cfg.layers} layers, {time.time() - t0:.0f}s",
                  flush=True)
        np.savez_compressed(os.path.join(HERE, f"{name}.npz"), **out)


if __name__ == "__main__":
    main(sys.argv[1:] or WORKLOADS)
