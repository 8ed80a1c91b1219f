#!/usr/bin/env python3
"""Throughput of one rank's TSP layer share on one MI355X.

A step is one tsp_layer_shard call: RMSNorm, D attention shards (QKV
projection, zigzag causal flash attention against the gathered K/V, O
projection accumulated in place), RMSNorm, D MLP shards (W1/W3 with SwiGLU,
W2 accumulated in place), residuals, with the other ranks' shards and K/V
rows streamed through the side-stream slots.  Inputs are resident in HBM
before the timed region; the other ranks' K/V rows (the all-gather's
payload) are produced beforehand with tsp_kv_shard and are not timed.  The
same steps replayed from a captured HIP graph are reported beside them
("other_launch"); --graph swaps the two.

Default workload: the 7B shape (h 4096, 32 heads x 128, SwiGLU 11008) at
S = 65536, fold D = 8, rank 3 (8192 local tokens in two zigzag chunks).

Prints one JSON line.  value = algorithmic TFLOP/s of the layer share:
F = 8 T h^2 + 6 T h F + 4 h P, P = causal (query, key) pairs of the rank.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)

METRIC = "TFLOP/s and tokens/s per TSP layer shard (7B shape), % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# The sources whose change voids the committed HBM counters: the kernels, and
# the host code that decides the launches (tile choice, shards per launch).
KERNEL_SRCS = [os.path.join(ROOT, "folded_tensor_sequence_rank_amd", "csrc", f)
               for f in ("tsp_kernels.hip", "tsp_api.cpp")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="7b_s64k")
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=32,
                    help="local rows of the rank's second chunk the oracle computes")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the headline steps only, launched eagerly: no graph, no second K/V "
                         "path, no clock-probe pass (for counter runs, which serialise every dispatch)")
    ap.add_argument("--mlp-backward", action="store_true",
                    help="time the MLP half's backward (tsp_mlp_shard_backward) instead of the layer")
    ap.add_argument("--attn-backward", action="store_true",
                    help="time the attention core's backward for one head group instead")
    ap.add_argument("--layer-backward", action="store_true",
                    help="time the whole layer's backward of one rank (both parts) instead")
    ap.add_argument("--recompute-attn", action="store_true",
                    help="with --layer-backward: recompute each head group's forward attention in the "
                         "backward instead of taking what tsp_attn_shard_save kept")
    ap.add_argument("--graph", action="store_true",
                    help="time the layer call replayed as a captured HIP graph instead of launched "
                         "eagerly (both are reported either way)")
    ap.add_argument("--kv-stream", action="store_true",
                    help="headline with the other ranks' K/V copied through the side-stream slots "
                         "(TSP_F_KV_STREAM) instead of read in place; both are reported either way")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first copy a buffer of this many MiB three times (a kernel of known "
                         "traffic for scaling HBM counters)")
    return ap.parse_args()


def flops_per_step(cfg, r):
    """Algorithmic FLOPs of each kernel class in one layer share (all its
    launches together): D QKV projections and D head-group attentions; the O
    and W2 projections over all shards (however they are grouped into
    launches); D W1/W3 projections."""
    from folded_tensor_sequence_rank_amd import tsp
    B = cfg.batch
    T, h, D, F = B * cfg.local_tokens, cfg.hidden, cfg.fold, cfg.ffn
    hk = cfg.kv_heads * cfg.head_dim  # K and V columns of the whole layer
    # causal (query, key) pairs of the rank's queries: key p' <= query p
    pos = tsp.zigzag_positions(cfg.seq, D, r)
    pairs = B * int((pos + 1).sum())  # per head, over the micro-batch
    return {"qkv": 2 * T * h * (h + 2 * hk), "attn": 4 * h * pairs, "oproj": 2 * T * h * h,
            "w13": 2 * T * 2 * F * h, "w2": 2 * T * F * h}


def bytes_per_launch(cfg):
    es = 2 if cfg.dtype == "bf16" else 4
    T, h = cfg.batch * cfg.local_tokens, cfg.hidden
    return {"rmsnorm": 2 * T * h * es + h * es}


def kernel_hash():
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None once the kernel or launch source has changed since the counters were
    taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


class ClockSampler:
    """Samples the graphics clock amdsmi reports (MHz, through
    torch.cuda.clock_rate) on a host thread while the timed steps run; None
    where the query is unavailable.  On this chip it reads the configured
    clock, not the one the power limit lets the kernels run at: the effective
    clock comes from the library's clock probe (effective_clock_mhz)."""

    def __init__(self):
        import threading
        self.samples = []
        self.stop = threading.Event()
        self.th = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        import torch
        try:
            while not self.stop.is_set():
                self.samples.append(float(torch.cuda.clock_rate(0)))
                time.sleep(0.002)
        except Exception:  # noqa: BLE001 - no clock query on this host
            pass

    def __enter__(self):
        self.th.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.th.join(timeout=5)

    def summary(self):
        v = sorted(x for x in self.samples if x > 0)
        if not v:
            return None
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1], "samples": len(v)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, r, rows):
    """The oracle, as it stands, on a bounded sample of the same workload:
    layer_rows for `rows` local rows of the rank's second chunk (with the
    rotary embedding and K/V heads of the workload).  The K/V projection of
    every position those rows attend to is part of that call; it is timed
    again on its own (the oracle's own steps: RMSNorm, n1 W_K rotated, n1 W_V,
    once per query head as multihead_causal forms them) so that the rank's
    own share can be reported without it."""
    import numpy as np
    import oracle.tsp_oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=os.cpu_count())
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    pos = O.zigzag_positions(cfg.seq, cfg.fold, r)[cfg.chunk: cfg.chunk + rows]
    pmax = int(pos.max()) + 1
    x = synth.gen_x_rows(cfg, 0, pmax)
    w = synth.gen_weights(cfg)
    reps = 3  # about 10 s of oracle work on the host cores
    t0 = time.perf_counter()
    for _ in range(reps):
        O.layer_rows(x, w, cfg.n_heads, cfg.eps, pos, cfg.rope_theta)
    dt = (time.perf_counter() - t0) / reps
    H, d, h, F = cfg.n_heads, cfg.head_dim, cfg.hidden, cfg.ffn
    grp = H // cfg.kv_heads
    allpos = np.arange(pmax)
    t0 = time.perf_counter()
    for _ in range(reps):
        n1 = O.rmsnorm(np.asarray(x[:pmax], np.float64), w.g1, cfg.eps)
        for t in range(H):
            kc = slice((t // grp) * d, (t // grp + 1) * d)
            O.rope(n1 @ np.asarray(w.wk[:, kc], np.float64), allpos, cfg.rope_theta)
            n1 @ np.asarray(w.wv[:, kc], np.float64)
    dkv = (time.perf_counter() - t0) / reps
    pairs = int(np.sum(pos + 1))
    # algorithmic FLOPs of the sample, counted as the GPU's are: Q and O of the
    # rows, K and V (Hkv heads) of every position they attend to, causal pairs,
    # the MLP of the rows
    kv_alg = 2 * 2 * pmax * h * cfg.kv_heads * d
    share_alg = 2 * rows * h * h + 4 * h * pairs + 2 * rows * h * h + 6 * rows * h * F
    # what the oracle executes: it forms K and V once per query head
    kv_exec = 2 * 2 * pmax * h * H * d
    share_s = max(dt - dkv, 1e-9)
    return {"value": round((kv_alg + share_alg) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt * reps, 3), "cpu": cpu_model(),
            "kv_projection_s": round(dkv, 4), "rank_share_s": round(share_s, 4),
            "rank_share_tflops": round(share_alg / share_s / 1e12, 6),
            "executed_tflops": round((kv_exec + share_alg) / dt / 1e12, 6),
            "sample": (f"{cfg.name}, rank {r}: fp64 numpy oracle layer_rows (rotary theta "
                       f"{cfg.rope_theta}, {cfg.kv_heads} K/V heads) for the first {rows} local rows "
                       f"of the second zigzag chunk (positions {int(pos[0])}..{int(pos[-1])}), "
                       f"including the K/V projection of all {pmax} positions they attend to, run "
                       f"{reps} times; value = the sample's algorithmic FLOPs (counted as the GPU's) / "
                       f"mean wall time; kv_projection_s = that projection alone, timed separately "
                       f"with the oracle's steps; rank_share_s = the rest")}


def mlp_backward_bench(args):
    """The MLP half's backward for one rank's rows at the workload's shape:
    algorithmic FLOPs 12*T*h*F (twice the forward's), plus 4*T*h*F to
    recompute n2 W1 and n2 W3, which the call does rather than store them."""
    import numpy as np
    import torch

    import synth
    from folded_tensor_sequence_rank_amd import tsp
    from gpu_harness import layer_dev, to_dev

    cfg = synth.get_config(args.workload)
    r = cfg.ranks[0] if args.rank is None else args.rank
    torch.cuda.set_device(0)
    D, h, Fs = cfg.fold, cfg.hidden, cfg.ffn // cfg.fold
    L = layer_dev(cfg, synth.gen_weights(cfg))
    pos = tsp.zigzag_positions(cfg.seq, D, r)
    x1 = to_dev(np.concatenate([synth.gen_rows(cfg, pos, seq_index=b) for b in range(cfg.batch)]), cfg)
    dout = to_dev(np.concatenate([synth.gen_rows(cfg, pos, layer=7, seq_index=b)
                                  for b in range(cfg.batch)]), cfg)
    dims = tsp.make_dims(cfg, r)
    ws = torch.empty(tsp.workspace_bytes(dims, tsp.TSP_WS_MLP_BWD), dtype=torch.uint8, device="cuda")
    dx1 = torch.empty_like(x1)
    dg2 = torch.empty(h, dtype=torch.float32, device="cuda")
    dw = [torch.empty(3 * Fs * h, dtype=torch.float32, device="cuda") for _ in range(D)]
    run = lambda: tsp.tsp_mlp_shard_backward(dims, x1, L.g2, L.w_mlp, dout, dx1, dg2, dw, ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    T = cfg.batch * cfg.local_tokens
    f_alg = 12 * T * h * cfg.ffn
    tflops = f_alg / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "TFLOP/s of the MLP half's backward per TSP layer shard (7B shape)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "rank": r, "batch": cfg.batch, "local_tokens": T},
        "frac_of_peak": round(tflops / (PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS), 4),
        "flops_per_step": f_alg, "recompute_flops_per_step": 4 * T * h * cfg.ffn}), flush=True)


def attn_backward_bench(args):
    """The attention core's backward for one head group (H/D query heads) of
    one rank's rows at the workload's shape.  Algorithmic FLOPs 8*d per
    (query, visible key) pair and head: dP = dO V^T, dV = P^T dO, dQ = dS K,
    dK = dS^T Q.  The call also recomputes 10*d per pair: the forward (scores
    and P V) for the log-sum-exp, and the scores in both backward kernels plus
    dP in the dQ kernel."""
    import torch

    import synth
    from folded_tensor_sequence_rank_amd import tsp

    cfg = synth.get_config(args.workload)
    r = cfg.ranks[0] if args.rank is None else args.rank
    torch.cuda.set_device(0)
    D, d, S, Bn = cfg.fold, cfg.head_dim, cfg.seq, cfg.batch
    T = S // D
    Hd, Hkd = cfg.n_heads // D, cfg.kv_heads // D
    g = torch.Generator(device="cuda")
    g.manual_seed(1234 + r)
    bf = torch.bfloat16
    q = torch.randn((Hd, Bn * T, d), generator=g, device="cuda").to(bf)
    kv = torch.randn((2 * Hkd * Bn * S * d,), generator=g, device="cuda").to(bf)
    do = torch.randn((Bn * T, Hd * d), generator=g, device="cuda").to(bf)
    dq = torch.empty((Hd, Bn * T, d), device="cuda")
    dk = torch.empty((Hkd, Bn * S, d), device="cuda")
    dv = torch.empty((Hkd, Bn * S, d), device="cuda")
    dims = tsp.make_dims(cfg, r)
    ws = torch.empty(tsp.workspace_bytes(dims, tsp.TSP_WS_ATTN_BWD), dtype=torch.uint8, device="cuda")
    run = lambda: tsp.tsp_attn_core_backward(dims, q, kv, do, dq, dk, dv, ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    pairs = int((tsp.zigzag_positions(S, D, r) + 1).sum())
    f_alg = 8 * d * pairs * Hd * Bn
    tflops = f_alg / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "TFLOP/s of the attention core's backward per head group (7B shape)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "rank": r, "batch": Bn, "local_tokens": Bn * T, "heads": Hd,
                   "kv_heads": Hkd},
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": f_alg, "recompute_flops_per_step": 10 * d * pairs * Hd * Bn}), flush=True)


def layer_backward_bench(args):
    """The whole layer's backward for one rank at the workload's shape: part 1
    (MLP half, then per head group the forward attention recomputed, dA and
    dW_O, the attention core's gradients) and part 2 (dn1 through W_Q/K/V,
    the partial dW_QKV, RMSNorm-1), timed together; the dK/dV exchange
    between them (a collective on D GPUs) is not.  Its input, the summed
    dK/dV of the rank's rows, is synthetic here.  Algorithmic FLOPs: twice
    the forward's projections and MLP (data and weight gradients,
    2 * (8 T h^2 + 6 T h F) at one K/V head per query head) and 8 d per
    (query, visible key) pair and head (dP, dV, dQ, dK).  The recomputation
    (S and dP in the dQ kernel, the MLP's and QKV's projections, the norms,
    and with --recompute-attn the forward attention) is reported apart.  By
    default the forward is tsp_attn_shard_save, whose attention output and
    softmax normalisers the backward takes."""
    import numpy as np
    import torch

    import synth
    from folded_tensor_sequence_rank_amd import tsp
    from gpu_harness import RankRun, fill_kv, layer_dev, new_kv, to_dev

    cfg = synth.get_config(args.workload)
    r = cfg.ranks[0] if args.rank is None else args.rank
    torch.cuda.set_device(0)
    D, h, d, H = cfg.fold, cfg.hidden, cfg.head_dim, cfg.n_heads
    B, T = cfg.batch, cfg.local_tokens
    BT, BS = B * T, B * cfg.seq
    Hkv = cfg.kv_heads
    hs, Fs, ks = h // D, cfg.ffn // D, Hkv * d // D
    L = layer_dev(cfg, synth.gen_weights(cfg))
    xs = [to_dev(np.concatenate([synth.gen_rows(cfg, tsp.zigzag_positions(cfg.seq, D, q), seq_index=b)
                                 for b in range(B)]), cfg) for q in range(D)]
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv)
    x = xs[r]
    xs = None
    saved = not args.recompute_attn
    if saved:
        x1, a_saved, lse_saved = RankRun(cfg, r).attn_save(x, L, kv)
    else:
        x1, a_saved, lse_saved = RankRun(cfg, r).attn(x, L, kv), None, None
    dout = to_dev(np.concatenate([synth.gen_rows(cfg, tsp.zigzag_positions(cfg.seq, D, r), layer=7, seq_index=b)
                                  for b in range(B)]), cfg)
    dims = tsp.make_dims(cfg, r)
    f32 = dict(dtype=torch.float32, device="cuda")
    ws1 = torch.empty(tsp.workspace_bytes(dims, tsp.TSP_WS_LAYER_BWD), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(tsp.workspace_bytes(dims, tsp.TSP_WS_LAYER_BWD_FINISH), dtype=torch.uint8, device="cuda")
    dx1, dx = torch.empty_like(x), torch.empty_like(x)
    dg1, dg2 = torch.empty(h, **f32), torch.empty(h, **f32)
    dw_mlp = [torch.empty(3 * Fs * h, **f32) for _ in range(D)]
    dw_o = [torch.empty(h * hs, **f32) for _ in range(D)]
    dw_qkv = [torch.empty((hs + 2 * ks) * h, **f32) for _ in range(D)]
    dq = torch.empty(H * BT * d, **f32)
    dkv = torch.empty(2 * Hkv * BS * d, **f32)
    g = torch.Generator(device="cuda")
    g.manual_seed(4321)
    dkv_own = torch.randn(2 * Hkv * BT * d, generator=g, **f32) * 1e-2

    def step():
        tsp.tsp_layer_shard_backward(dims, x, x1, L.g1, L.w_attn, kv, L.g2, L.w_mlp, dout, dx1, dg2, dw_mlp, dw_o,
                                     dq, dkv, ws1, attn_saved=a_saved, lse_saved=lse_saved)
        tsp.tsp_layer_shard_backward_finish(dims, x, L.g1, L.w_attn, dx1, dq, dkv_own, dx, dg1, dw_qkv, ws2)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record()
    for i in range(args.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    pairs = B * int((tsp.zigzag_positions(cfg.seq, D, r) + 1).sum())
    proj = 2 * BT * h * (h + 2 * Hkv * d) + 2 * BT * h * h + 6 * BT * h * cfg.ffn
    f_alg = 2 * proj + 8 * d * pairs * H
    recompute = ((0 if saved else 4 * d * pairs * H)  # forward attention for O and the log-sum-exp
                 + 4 * d * pairs * H        # S and dP again in the dQ kernel
                 + 4 * BT * h * cfg.ffn     # n2 W1 and n2 W3
                 + 2 * BT * h * (h + 2 * Hkv * d))  # Q and the rank's own K/V rows
    tflops = f_alg / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "TFLOP/s of one rank's whole-layer backward (7B shape)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "step_ms": {"median": round(per[len(per) // 2], 4), "min": round(per[0], 4), "max": round(per[-1], 4)},
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "rank": r, "batch": B, "local_tokens": BT,
                   "attention": "saved by the forward" if saved else "recomputed"},
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": f_alg, "recompute_flops_per_step": recompute,
        "executed_tflops": round((f_alg + recompute) / (ms * 1e-3) / 1e12, 2)}), flush=True)


def hbm_copy_rate(mib=1024, reps=5):
    """A device-to-device copy of `mib` MiB (the runtime's copy kernel) timed
    with HIP events: bytes read plus bytes written per second, the measured
    counterpart of the 8 TB/s HBM figure against which the HBM-bound kernels'
    GB/s read."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"bytes_per_copy_read_and_written": 2 * n, "ms": round(ms, 4),
            "gbs": round(2 * n / (ms * 1e-3) / 1e9, 1), "peak_gbs": 8000.0}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the layer: the TSP path here runs on a "
              "single MI355X (one rank at its real shape); multi-GPU runs are not part of it.",
              file=sys.stderr)
        sys.exit(2)
    if args.mlp_backward:
        mlp_backward_bench(args)
        return
    if args.attn_backward:
        attn_backward_bench(args)
        return
    if args.layer_backward:
        layer_backward_bench(args)
        return

    import numpy as np
    import torch

    import synth
    from folded_tensor_sequence_rank_amd import tsp
    from gpu_harness import RankRun, fill_kv, layer_dev, new_kv, to_dev

    cfg = synth.get_config(args.workload)
    r = cfg.ranks[0] if args.rank is None else args.rank
    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    hbm = None if args.headline_only else hbm_copy_rate()
    t_setup = time.perf_counter()
    w = synth.gen_weights(cfg)
    L = layer_dev(cfg, w)
    del w
    xs = []
    for q in range(cfg.fold):
        pos = tsp.zigzag_positions(cfg.seq, cfg.fold, q)
        # sequence-major rows of every sequence of the micro-batch
        xs.append(to_dev(np.concatenate([synth.gen_rows(cfg, pos, seq_index=b)
                                         for b in range(cfg.batch)]), cfg))
    kv = new_kv(cfg)
    fill_kv(cfg, L, xs, kv, skip=r)
    x = xs[r]
    for q in range(cfg.fold):
        if q != r:
            xs[q] = None
    out = torch.empty_like(x)
    run = RankRun(cfg, r)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    runs = {"in_place": run, "kv_stream": RankRun(cfg, r, flags=tsp.TSP_F_KV_STREAM)}
    head = "kv_stream" if args.kv_stream else "in_place"
    warm = []
    for _ in range(args.warmup):
        t0 = time.perf_counter()
        runs[head].layer(x, L, kv, out)
        torch.cuda.synchronize()
        warm.append((time.perf_counter() - t0) * 1e3)
    est_ms = min(warm) if warm else 10.0  # a step's wall time, for sizing the clock probe

    # The layer call captured once into a HIP graph (its kernels, side-stream
    # copies and the events ordering them) and replayed per step: the same
    # launches without the host's per-launch cost between them.
    graphs = {}

    def capture(name):
        """The call captured into a graph whose replay writes what the eager
        call writes, bit for bit (checked)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            runs[name].layer(x, L, kv, out)
        torch.cuda.synchronize()
        runs[name].layer(x, L, kv, out)
        torch.cuda.synchronize()
        ref = out.clone()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "graph replay differs from the eager call"
        return g

    def timed(rr, probe=False, graph=None):
        """K steps bracketed by synchronisation, an event between steps; with
        probe, the clock probe runs on a second stream over ~90% of them.
        With graph, each step replays it instead of calling rr.layer.  The W
        warmup steps run right before, in the same launch mode, so that the
        timed steps do not start on a GPU that idled through the set-up."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        samples, khz = None, 0
        for _ in range(args.warmup):
            if graph is not None:
                graph.replay()
            else:
                rr.layer(x, L, kv, out)
        torch.cuda.synchronize()
        if probe:
            interval_us = 200
            n = int(min(4e6 / interval_us, max(8, est_ms * 1e3 * args.steps * 0.9 / interval_us)))
            samples = torch.zeros(2 * n, dtype=torch.int64, device="cuda")
            ps = torch.cuda.Stream()
            khz = tsp.tsp_clock_probe(samples, n, interval_us, stream=ps)
        ev[0].record()
        for i in range(args.steps):
            if graph is not None:
                graph.replay()
            else:
                rr.layer(x, L, kv, out)
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
        return ev[0].elapsed_time(ev[-1]) / args.steps, per, (samples, khz)

    # (counter runs, --headline-only, launch eagerly and time one mode only)
    use_graph = args.graph and not args.headline_only
    if use_graph:
        graphs[head] = capture(head)
    with ClockSampler() as clk:
        ms, step_times, _ = timed(runs[head], graph=graphs.get(head))
    assert torch.isfinite(out).all(), "non-finite output"
    # the other launch mode of the same steps, for comparison
    ms_alt, per_alt = None, None
    if not args.headline_only:
        ms_alt, per_alt, _ = timed(runs[head], graph=None if use_graph else capture(head))
    # The effective clock, from a second pass of the same steps with the clock
    # probe beside them.  Not during the timed steps: the probe's wave holds a
    # slot on one CU, which keeps a full-register workgroup off that CU (a
    # GEMM launch of exactly two rounds of 256 tiles then needs a third).
    eff_clock, other, ms_other, per_other = None, None, None, None
    if not args.headline_only:
        ms_probe, _, (samples, khz) = timed(runs[head], probe=True, graph=graphs.get(head))
        smp = samples.cpu().numpy().reshape(-1, 2)
        smp = smp[smp[:, 0] - smp[0, 0] <= ms_probe * args.steps * khz]  # inside the steps
        mhz = tsp.clock_mhz(smp, khz)
        eff_clock = None if mhz.size == 0 else {
            "median_mhz": round(float(np.median(mhz)), 1), "min_mhz": round(float(mhz.min()), 1),
            "max_mhz": round(float(mhz.max()), 1), "intervals": int(mhz.size), "interval_us": 200,
            "probe_pass_ms_per_step": round(ms_probe, 4),
            "source": "tsp_clock_probe: shader-clock cycles per wall-clock tick, one wave beside a second "
                      "pass of the steps (not the timed one)"}
        other = "kv_stream" if head == "in_place" else "in_place"
        for _ in range(args.warmup):
            runs[other].layer(x, L, kv, out)
        if use_graph:
            graphs[other] = capture(other)
        ms_other, per_other, _ = timed(runs[other], graph=graphs.get(other))

    T = cfg.batch * cfg.local_tokens
    f_alg = sum(flops_per_step(cfg, r).values())
    tflops = f_alg / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS

    def step_stats(per):
        v = sorted(per)
        return {"median": round(v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2]), 4),
                "min": round(v[0], 4), "max": round(v[-1], 4)}

    variant = None if other is None else {
        "path": other, "ms_per_step": round(ms_other, 4), "value": round(f_alg / (ms_other * 1e-3) / 1e12, 2),
        "frac_of_peak": round(f_alg / (ms_other * 1e-3) / 1e12 / peak, 4),
        "tokens_per_s": round(T / (ms_other * 1e-3), 1), "step_ms": step_stats(per_other)}

    kernels, roofline = {}, None
    if not args.no_profile:
        prun = RankRun(cfg, r, flags=tsp.TSP_F_PROFILE | (tsp.TSP_F_KV_STREAM if head == "kv_stream" else 0))
        prun.layer(x, L, kv, out)
        torch.cuda.synchronize()
        tsp.tsp_profile_read(reset=True)
        for _ in range(args.steps):
            prun.layer(x, L, kv, out)
        torch.cuda.synchronize()
        prof = tsp.tsp_profile_read(reset=True)
        fs = flops_per_step(cfg, r)
        by = bytes_per_launch(cfg)
        fl = {}  # FLOPs per launch of each class
        for k, (tot, n) in prof.items():
            if n == 0:
                continue
            avg = tot / n
            per_step = n / args.steps
            ent = {"ms_avg": round(avg, 5), "launches_per_step": per_step,
                   "ms_per_step": round(tot / args.steps, 4)}
            if k in fs:
                fl[k] = fs[k] / per_step
                ent["tflops"] = round(fl[k] / (avg * 1e-3) / 1e12, 1)
            if k in by:
                ent["gbs"] = round(by[k] / (avg * 1e-3) / 1e9, 1)
            kernels[k] = ent
        dom = max((k for k in kernels if k in fl), key=lambda k: kernels[k]["ms_per_step"])
        ach = fl[dom] / (kernels[dom]["ms_avg"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                    "flops_per_launch": int(fl[dom]), "traffic": traffic_for(dom)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, r, args.cpu_rows)

    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "hidden": cfg.hidden, "heads": cfg.n_heads,
                   "head_dim": cfg.head_dim, "ffn": cfg.ffn, "seq": cfg.seq, "fold": cfg.fold,
                   "rank": r, "batch": cfg.batch, "local_tokens": T,
                   "kv_heads": cfg.kv_heads, "rope_theta": cfg.rope_theta,
                   "parallelism": "tsp-rank-share"},
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "frac_of_peak": round(tflops / peak, 4),
        "step_ms": step_stats(step_times),
        "kv_path": head,
        "kv_variant": variant,
        "launch": "hip_graph" if use_graph else "eager",
        "other_launch": None if ms_alt is None else {
            "launch": "eager" if use_graph else "hip_graph", "ms_per_step": round(ms_alt, 4),
            "value": round(f_alg / (ms_alt * 1e-3) / 1e12, 2), "step_ms": step_stats(per_alt)},
        "flops_per_step": f_alg,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "effective_clock_mhz": eff_clock,
        "gpu_clock_configured": clk.summary(),
        "hbm_copy": hbm,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
