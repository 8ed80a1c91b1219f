"""CPU oracle for one rank of a folded tensor+sequence parallel (TSP) layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module; only tests, the package's smoke check and the benchmark's CPU-baseline
leg do.  It is plain numpy in float64, written for a reader to check against
the source by eye, and it shares no code with the HIP library.

Source: "Folding Tensor and Sequence Parallelism for Memory-Efficient
Transformer Training & Inference" (gist.science summary), section 2
"Metodologia: TSP" and its list of main design components.  The method
re-organises WHERE the work of an ordinary pre-norm transformer layer runs:
every rank keeps 1/D of the weights and 1/D of the tokens (unified
sharding), attention weight shards are broadcast one by one, K/V are
all-gathered along the sequence, and gated-MLP shards travel round a ring
while each rank sums its partial outputs locally.  None of that changes the
result, so the oracle is the unsharded layer, restricted to one rank's rows.

Readings where the pages are silent (each is listed in the design notes):
  * zigzag: the sequence is cut into 2D equal chunks; rank r holds chunks r
    and 2D-1-r, chunk r first.  (Section 2, attention layers, "zigzag
    partitioning"; the tiny workload's rank 1 of 4 holding chunks 1 and 6
    fixes the rule.)
  * weight shards are head groups: shard j holds heads [j*H/D, (j+1)*H/D) of
    W_Q, W_K, W_V (output columns) and the matching rows of W_O; MLP shard j
    holds columns [j*F/D, (j+1)*F/D) of W1 and W3 and those rows of W2.
  * layer: pre-norm RMSNorm (eps inside the root), causal softmax attention
    with scale 1/sqrt(d) and the diagonal included, residual, RMSNorm, SwiGLU
    MLP silu(n W1) * (n W3) then W2, residual.  No bias, no dropout.  By
    default no positional encoding and every head has its own K/V (the
    pages' setting).
  * extensions the pages do not describe, off by default: grouped-query
    attention (W_K, W_V with Hkv*d columns; query head t reads K/V head
    t // (H/Hkv); a K/V shard is K/V head group j), and the rotary position
    embedding of RoFormer (Su et al. 2021, section 3.2) applied to Q and K at
    each token's global position, pair (2i, 2i+1) of a head turned by
    p * theta^(-2i/d).

Functions that carry a pin in tests/test_oracle.py are marked "pinned by".
"""
from __future__ import annotations

import math
from typing import Iterable, List, Sequence

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# Zigzag token layout (section 2, attention layers: zigzag partitioning)
# --------------------------------------------------------------------------

def zigzag_chunks(D: int, r: int):
    """The two chunk indices rank r holds out of 2D: r and 2D-1-r.

    Pinned by: the tiny workload's statement (D=4, r=1 -> chunks 1 and 6),
    partition of the sequence, equal causal work per rank."""
    return (r, 2 * D - 1 - r)


def zigzag_positions(S: int, D: int, r: int) -> np.ndarray:
    """Global positions of rank r's local rows, in local order."""
    if S % (2 * D):
        raise ValueError("S must be a multiple of 2D")
    C = S // (2 * D)
    a, b = zigzag_chunks(D, r)
    return np.concatenate([np.arange(a * C, (a + 1) * C), np.arange(b * C, (b + 1) * C)]).astype(np.int64)


def unzigzag(parts: Sequence[np.ndarray], S: int, D: int) -> np.ndarray:
    """Place every rank's local rows back at their global positions."""
    out = np.empty((S,) + parts[0].shape[1:], dtype=parts[0].dtype)
    for r, p in enumerate(parts):
        out[zigzag_positions(S, D, r)] = p
    return out


def causal_pairs(S: int, D: int, r: int) -> int:
    """Number of (query, key) pairs with key <= query among rank r's queries:
    the causal attention work the rank does.  Counted directly."""
    return int(np.sum(zigzag_positions(S, D, r) + 1))


# --------------------------------------------------------------------------
# Layer pieces (textbook definitions)
# --------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g, row-wise.  Pinned by torch rms_norm."""
    x = np.asarray(x, F64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, F64)


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z).  Pinned by torch silu."""
    return z / (1.0 + np.exp(-z))


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary position embedding (RoFormer, section 3.2) of one head's rows.

    x [R, d], pos [R] positions.  The pair of dims (2i, 2i+1) of row p is
    turned counter-clockwise by p * theta^(-2i/d):
    (u, v) -> (u cos a - v sin a, u sin a + v cos a).  theta == 0 returns x.
    Pinned by transformers' Llama rotary embedding (which pairs dims i and
    i + d/2: the same map up to a fixed permutation of the head dims) and by
    the relative-position property of rotated dot products."""
    x = np.asarray(x, F64)
    if not theta:
        return x
    d = x.shape[1]
    freq = float(theta) ** (-2.0 * np.arange(d // 2) / d)
    a = np.asarray(pos, F64)[:, None] * freq[None, :]
    c, s = np.cos(a), np.sin(a)
    u, v = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = u * c - v * s
    out[:, 1::2] = u * s + v * c
    return out


def kv_heads(w, n_heads: int) -> int:
    """Hkv, from the width of W_K (h columns for ordinary multi-head attention)."""
    d = w.wq.shape[1] // n_heads
    return w.wk.shape[1] // d


def multihead_causal(n1: np.ndarray, rows: np.ndarray, w, n_heads: int, rope_theta: float) -> np.ndarray:
    """Concatenated head outputs A [len(rows), h] of causal attention for the
    queries at global positions `rows`, n1 [>= max(rows)+1, h] being the
    normalised input of every position.  Query head t uses columns
    [t*d, (t+1)*d) of W_Q and K/V head t // (H/Hkv).  Pinned against torch
    scaled_dot_product_attention (enable_gqa) and the Llama decoder layer."""
    h = w.wq.shape[1]
    d = h // n_heads
    grp = n_heads // kv_heads(w, n_heads)
    P = n1.shape[0]
    q = n1[rows] @ np.asarray(w.wq, F64)
    a = np.empty((rows.size, h), F64)
    for t in range(n_heads):
        c = slice(t * d, (t + 1) * d)
        kc = slice((t // grp) * d, (t // grp + 1) * d)
        k_t = rope(n1 @ np.asarray(w.wk[:, kc], F64), np.arange(P), rope_theta)
        v_t = n1 @ np.asarray(w.wv[:, kc], F64)
        a[:, c] = causal_attention(rope(q[:, c], rows, rope_theta), rows, k_t, v_t)
    return a


def causal_attention(q: np.ndarray, qpos: np.ndarray, k: np.ndarray, v: np.ndarray,
                     block: int = 128) -> np.ndarray:
    """Softmax attention of queries at global positions qpos against keys
    0..max(qpos); key j is visible to a query at p iff j <= p.

    q [R, d]; k, v [P, d] indexed by global position.  Scores are scaled by
    1/sqrt(d).  Query blocks bound the memory (no S x S matrix).
    Pinned by torch scaled_dot_product_attention(is_causal=True), a pure
    Python double loop, and the first-position and uniform-score cases."""
    q = np.asarray(q, F64)
    qpos = np.asarray(qpos, np.int64)
    d = q.shape[1]
    out = np.empty_like(q)
    scale = 1.0 / math.sqrt(d)
    for s in range(0, q.shape[0], block):
        qb, pb = q[s:s + block], qpos[s:s + block]
        kmax = int(pb.max()) + 1
        sc = (qb @ np.asarray(k[:kmax], F64).T) * scale
        sc[np.arange(kmax)[None, :] > pb[:, None]] = -np.inf
        m = sc.max(axis=1, keepdims=True)
        e = np.exp(sc - m)
        out[s:s + block] = (e @ np.asarray(v[:kmax], F64)) / e.sum(axis=1, keepdims=True)
    return out


def swiglu_mlp(n: np.ndarray, w1, w3, w2) -> np.ndarray:
    """(silu(n W1) * (n W3)) W2: the gated MLP (section 2, gated MLP layers)."""
    return (silu(n @ np.asarray(w1, F64)) * (n @ np.asarray(w3, F64))) @ np.asarray(w2, F64)


# --------------------------------------------------------------------------
# The unsharded layer, restricted to chosen rows
# --------------------------------------------------------------------------

def layer_rows(x_full: np.ndarray, w, n_heads: int, eps: float, rows: Iterable[int],
               rope_theta: float = 0.0) -> np.ndarray:
    """Output of one unsharded pre-norm layer at global positions `rows`.

    x_full must hold at least rows 0..max(rows) (causal attention needs every
    earlier position's K/V).  Steps: n1 = RMSNorm(x); Q, K, V = n1 W_{Q,K,V};
    per-head causal attention (Q and K rotated when rope_theta > 0);
    x1 = x + A W_O; n2 = RMSNorm(x1); out = x1 + SwiGLU(n2)."""
    rows = np.asarray(list(rows) if not isinstance(rows, np.ndarray) else rows, np.int64)
    x1 = attention_block_rows(x_full, w, n_heads, eps, rows, rope_theta)
    return mlp_block(x1, w, eps)


def layer_unsharded(x_full: np.ndarray, w, n_heads: int, eps: float,
                    rope_theta: float = 0.0) -> np.ndarray:
    return layer_rows(x_full, w, n_heads, eps, np.arange(x_full.shape[0]), rope_theta)


def attention_block_rows(x_full, w, n_heads, eps, rows, rope_theta: float = 0.0) -> np.ndarray:
    """x1 = x + Attn(RMSNorm(x)) W_O at `rows`: the attention half alone."""
    rows = np.asarray(rows, np.int64)
    pmax = int(rows.max()) + 1
    xs = np.asarray(x_full[:pmax], F64)
    n1 = rmsnorm(xs, w.g1, eps)
    a = multihead_causal(n1, rows, w, n_heads, rope_theta)
    return xs[rows] + a @ np.asarray(w.wo, F64)


def mlp_block(x1: np.ndarray, w, eps: float) -> np.ndarray:
    """out = x1 + SwiGLU(RMSNorm(x1)): the MLP half alone (row-local)."""
    x1 = np.asarray(x1, F64)
    return x1 + swiglu_mlp(rmsnorm(x1, w.g2, eps), w.w1, w.w3, w.w2)


def stack_rows(x_full: np.ndarray, ws: List, n_heads: int, eps: float, rows,
               rope_theta: float = 0.0) -> np.ndarray:
    """Output of a stack of layers at `rows`.  Every layer but the last is
    evaluated at all positions up to max(rows), since the next layer's
    attention reads them."""
    rows = np.asarray(rows, np.int64)
    pmax = int(rows.max()) + 1
    h = np.asarray(x_full[:pmax], F64)
    for w in ws[:-1]:
        h = layer_rows(h, w, n_heads, eps, np.arange(pmax), rope_theta)
    return layer_rows(h, ws[-1], n_heads, eps, rows, rope_theta)


def rank_share(x_full: np.ndarray, w, n_heads: int, eps: float, S: int, D: int, r: int,
               rope_theta: float = 0.0) -> np.ndarray:
    """Rank r's output rows, in its local (zigzag) order."""
    return layer_rows(x_full, w, n_heads, eps, zigzag_positions(S, D, r), rope_theta)


# --------------------------------------------------------------------------
# The sharded schedule, replayed literally (brute force, tiny sizes only)
# --------------------------------------------------------------------------

def fold_schedule(x_full: np.ndarray, w, n_heads: int, eps: float, D: int,
                  ring_order: bool = True, rope_theta: float = 0.0) -> List[np.ndarray]:
    """Run every rank's TSP schedule for one layer, rank by rank, and return
    each rank's local output rows.

    Attention (section 2, attention layers, broadcast schedule): for each
    broadcast iteration j the packed shard {W_Q, W_K, W_V, W_O} of head group
    j reaches every rank; each rank projects its own tokens; K and V are
    all-gathered along the sequence; each rank attends its local queries to
    the full K/V and adds its partial O-projection locally.  With the rotary
    embedding, each rank rotates its Q and K rows at the global positions it
    holds before the gather.
    MLP (section 2, gated MLP layers, ring schedule): at ring step t rank r
    holds shard (r + t) mod D of W1, W3, W2 and accumulates the partial
    output locally; no all-reduce is needed."""
    S, h = x_full.shape
    H = n_heads
    d = h // H
    hs = h // D
    ks = kv_heads(w, H) * d // D            # K/V columns per shard
    grp = hs // ks                          # query heads per K/V head
    F = w.w1.shape[1]
    Fs = F // D
    pos = [zigzag_positions(S, D, r) for r in range(D)]
    xr = [np.asarray(x_full[p], F64) for p in pos]
    n1 = [rmsnorm(x, w.g1, eps) for x in xr]
    y = [np.zeros((p.size, h), F64) for p in pos]

    def rot(m, p):                          # rotary embedding of every head of m
        return np.concatenate([rope(m[:, t * d:(t + 1) * d], p, rope_theta)
                               for t in range(m.shape[1] // d)], axis=1)

    for j in range(D):                      # broadcast iteration: shard of rank j
        cols = slice(j * hs, (j + 1) * hs)
        kcols = slice(j * ks, (j + 1) * ks)
        wq_j = np.asarray(w.wq[:, cols], F64)
        wk_j, wv_j = (np.asarray(m[:, kcols], F64) for m in (w.wk, w.wv))
        wo_j = np.asarray(w.wo[cols, :], F64)
        q = [rot(n @ wq_j, p) for n, p in zip(n1, pos)]   # local projections
        k_full = np.zeros((S, ks), F64)     # all-gather along the sequence
        v_full = np.zeros((S, ks), F64)
        for r in range(D):
            k_full[pos[r]] = rot(n1[r] @ wk_j, pos[r])
            v_full[pos[r]] = n1[r] @ wv_j
        for r in range(D):
            o = np.empty((pos[r].size, hs), F64)
            for t in range(hs // d):
                c = slice(t * d, (t + 1) * d)
                kc = slice((t // grp) * d, (t // grp + 1) * d)
                o[:, c] = causal_attention(q[r][:, c], pos[r], k_full[:, kc], v_full[:, kc])
            y[r] += o @ wo_j                # local partial O-projection
    x1 = [x + yy for x, yy in zip(xr, y)]
    n2 = [rmsnorm(x, w.g2, eps) for x in x1]
    out = []
    for r in range(D):
        acc = np.zeros_like(x1[r])
        for t in range(D):                  # ring step t
            j = (r + t) % D if ring_order else t
            fc = slice(j * Fs, (j + 1) * Fs)
            acc += swiglu_mlp(n2[r], w.w1[:, fc], w.w3[:, fc], w.w2[fc, :])
        out.append(x1[r] + acc)
    return out


def mlp_partials(n: np.ndarray, w, D: int) -> List[np.ndarray]:
    """The D per-shard partial MLP outputs of one rank (before summing)."""
    Fs = w.w1.shape[1] // D
    return [swiglu_mlp(n, w.w1[:, j * Fs:(j + 1) * Fs], w.w3[:, j * Fs:(j + 1) * Fs],
                       w.w2[j * Fs:(j + 1) * Fs, :]) for j in range(D)]


# --------------------------------------------------------------------------
# Work model (section 3, FLOPs: same per-device compute as TP and SP)
# --------------------------------------------------------------------------

def flops_rank(h: int, F: int, S: int, D: int, r: int) -> int:
    """Algorithmic FLOPs of rank r's layer share: QKV and O projections of its
    T tokens (8 T h^2), the SwiGLU MLP (6 T h F), and 4 h flops per causal
    (query, key) pair (scores and the weighted sum of values)."""
    T = S // D
    return 8 * T * h * h + 6 * T * h * F + 4 * h * causal_pairs(S, D, r)


def flops_unsharded(h: int, F: int, S: int) -> int:
    """FLOPs of the whole layer on one device, counted the same way."""
    return 8 * S * h * h + 6 * S * h * F + 4 * h * (S * (S + 1) // 2)


def rel_fro(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_F / ||ref||_F in float64."""
    a = np.asarray(a, F64)
    ref = np.asarray(ref, F64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / (den if den > 0 else 1.0))
