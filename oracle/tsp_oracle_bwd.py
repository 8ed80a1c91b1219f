"""CPU oracle of the backward pass of one TSP layer (gradients).

TEST INFRASTRUCTURE ONLY, like the forward oracle beside it: plain numpy in
float64, no code shared with the HIP library, imported only by tests.

The pages describe the forward schedules only (broadcast of attention
shards, K/V all-gather, ring of MLP shards; "Folding Tensor and Sequence
Parallelism ...", section 2), so the backward is a reading of our own, the
plainest one the forward supports:

  * the unsharded layer's gradients are the definition (hand-written chain
    rule below, pinned against torch autograd and finite differences);
  * each rank r computes, from its own zigzag rows, the input gradient of
    those rows and a PARTIAL gradient of every weight shard; the full weight
    gradient is the sum of the D partials (a reduce-scatter to each shard's
    owner replaces the forward broadcast / ring);
  * in the attention half, rank r's queries produce gradients for the K/V of
    every position they attended to; those partial dK/dV are summed at the
    owners of the positions (the reverse of the K/V all-gather) before each
    rank forms dW_K, dW_V and its input gradient.

Layer, as in the forward oracle: n1 = RMSNorm(x; g1); per head Q, K, V
(rotary embedding on Q and K when theta > 0; grouped K/V heads); causal
softmax attention; x1 = x + A W_O; n2 = RMSNorm(x1; g2);
out = x1 + (silu(n2 W1) * (n2 W3)) W2.
"""
from __future__ import annotations

import math
from types import SimpleNamespace

import numpy as np

from oracle.tsp_oracle import (F64, causal_attention, kv_heads, rmsnorm, rope, silu,
                               unzigzag, zigzag_positions)


def rmsnorm_backward(x, g, eps, dy):
    """Gradients of y = x * r * g, r = (mean(x^2) + eps)^(-1/2) per row:
    dx = r * u - x * r^3 * <u, x> / h with u = dy * g, and dg = sum_rows dy * x * r."""
    x = np.asarray(x, F64)
    g = np.asarray(g, F64)
    dy = np.asarray(dy, F64)
    h = x.shape[-1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    u = dy * g
    dx = r * u - x * r ** 3 * np.sum(u * x, axis=-1, keepdims=True) / h
    dg = np.sum(dy * x * r, axis=0)
    return dx, dg


def swiglu_backward(n, w1, w3, w2, dout):
    """Gradients of out = (silu(n W1) * (n W3)) W2 with respect to n, W1, W3, W2.
    silu'(a) = sigmoid(a) (1 + a (1 - sigmoid(a)))."""
    n = np.asarray(n, F64)
    w1, w3, w2 = (np.asarray(m, F64) for m in (w1, w3, w2))
    dout = np.asarray(dout, F64)
    a, b = n @ w1, n @ w3
    sg = 1.0 / (1.0 + np.exp(-a))
    s = a * sg
    gm = s * b
    dgm = dout @ w2.T
    da = dgm * b * sg * (1.0 + a * (1.0 - sg))
    db = dgm * s
    return da @ w1.T + db @ w3.T, n.T @ da, n.T @ db, gm.T @ dout


def causal_attention_backward(q, qpos, k, v, do):
    """Gradients of o = softmax(q k^T / sqrt(d), keys j <= qpos) v.
    q [R, d] at positions qpos; k, v [P, d] by position.  With P the
    probabilities: dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(P dP)),
    dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).  dk, dv cover positions
    0..P-1 (rows past max(qpos) stay zero)."""
    q, k, v, do = (np.asarray(t, F64) for t in (q, k, v, do))
    qpos = np.asarray(qpos, np.int64)
    d = q.shape[1]
    scale = 1.0 / math.sqrt(d)
    kmax = int(qpos.max()) + 1
    sc = (q @ k[:kmax].T) * scale
    sc[np.arange(kmax)[None, :] > qpos[:, None]] = -np.inf
    p = np.exp(sc - sc.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = do @ v[:kmax].T
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dv[:kmax] = p.T @ do
    dk[:kmax] = ds.T @ q * scale
    return ds @ k[:kmax] * scale, dk, dv


def layer_backward(x, w, n_heads, eps, dout, rope_theta=0.0):
    """Gradients of the unsharded layer over a whole sequence x [S, h], given
    dout [S, h].  Returns (dx, grads) with grads g1, wq, wk, wv, wo, g2, w1, w3, w2."""
    x = np.asarray(x, F64)
    dout = np.asarray(dout, F64)
    S, h = x.shape
    d = w.wq.shape[1] // n_heads
    grp = n_heads // kv_heads(w, n_heads)
    pos = np.arange(S)
    wq, wk, wv, wo = (np.asarray(m, F64) for m in (w.wq, w.wk, w.wv, w.wo))
    # forward, keeping what the backward needs
    n1 = rmsnorm(x, w.g1, eps)
    q_all, k_all, v_all = n1 @ wq, n1 @ wk, n1 @ wv
    a = np.empty((S, h), F64)
    for t in range(n_heads):
        c = slice(t * d, (t + 1) * d)
        kc = slice((t // grp) * d, (t // grp + 1) * d)
        a[:, c] = causal_attention(rope(q_all[:, c], pos, rope_theta), pos,
                                   rope(k_all[:, kc], pos, rope_theta), v_all[:, kc])
    x1 = x + a @ wo
    n2 = rmsnorm(x1, w.g2, eps)
    # MLP half
    dn2, dw1, dw3, dw2 = swiglu_backward(n2, w.w1, w.w3, w.w2, dout)
    dx1n, dg2 = rmsnorm_backward(x1, w.g2, eps, dn2)
    dx1 = dout + dx1n
    # attention half
    dwo = a.T @ dx1
    da = dx1 @ wo.T
    dq_all = np.zeros_like(q_all)
    dk_all = np.zeros_like(k_all)
    dv_all = np.zeros_like(v_all)
    for t in range(n_heads):
        c = slice(t * d, (t + 1) * d)
        kc = slice((t // grp) * d, (t // grp + 1) * d)
        dq, dk, dv = causal_attention_backward(rope(q_all[:, c], pos, rope_theta), pos,
                                               rope(k_all[:, kc], pos, rope_theta), v_all[:, kc],
                                               da[:, c])
        # the rotation is orthogonal: its backward turns by the opposite angle
        dq_all[:, c] = rope(dq, -pos, rope_theta)
        dk_all[:, kc] += rope(dk, -pos, rope_theta)
        dv_all[:, kc] += dv
    dn1 = dq_all @ wq.T + dk_all @ wk.T + dv_all @ wv.T
    dxn, dg1 = rmsnorm_backward(x, w.g1, eps, dn1)
    grads = SimpleNamespace(g1=dg1, wq=n1.T @ dq_all, wk=n1.T @ dk_all, wv=n1.T @ dv_all, wo=dwo,
                            g2=dg2, w1=dw1, w3=dw3, w2=dw2)
    return dx1 + dxn, grads


def fold_schedule_backward(x, w, n_heads, eps, dout, D, rope_theta=0.0):
    """The backward reading above replayed rank by rank: each rank works on
    its own zigzag rows, takes the other ranks' forward K/V rows and the
    reduce-scattered dK/dV of its own rows, and produces its rows' input
    gradient and a partial gradient of every weight.  Returns (dx per rank
    in local order, partial grads per rank)."""
    x = np.asarray(x, F64)
    dout = np.asarray(dout, F64)
    S, h = x.shape
    d = w.wq.shape[1] // n_heads
    hk = kv_heads(w, n_heads) * d
    grp = n_heads // kv_heads(w, n_heads)
    pos = [zigzag_positions(S, D, r) for r in range(D)]
    wq, wk, wv, wo = (np.asarray(m, F64) for m in (w.wq, w.wk, w.wv, w.wo))
    xr = [x[p] for p in pos]
    n1 = [rmsnorm(t, w.g1, eps) for t in xr]
    # forward per rank; K/V all-gathered by position
    q = [rope_heads(n @ wq, p, d, rope_theta) for n, p in zip(n1, pos)]
    k_full = np.zeros((S, hk), F64)
    v_full = np.zeros((S, hk), F64)
    for r in range(D):
        k_full[pos[r]] = rope_heads(n1[r] @ wk, pos[r], d, rope_theta)
        v_full[pos[r]] = n1[r] @ wv
    a = []
    for r in range(D):
        ar = np.empty((pos[r].size, h), F64)
        for t in range(n_heads):
            c = slice(t * d, (t + 1) * d)
            kc = slice((t // grp) * d, (t // grp + 1) * d)
            ar[:, c] = causal_attention(q[r][:, c], pos[r], k_full[:, kc], v_full[:, kc])
        a.append(ar)
    x1 = [t + ar @ wo for t, ar in zip(xr, a)]
    n2 = [rmsnorm(t, w.g2, eps) for t in x1]
    dr = [dout[p] for p in pos]
    parts = []
    dx1 = []
    for r in range(D):   # MLP half: local; weight gradients are partial
        dn2, dw1, dw3, dw2 = swiglu_backward(n2[r], w.w1, w.w3, w.w2, dr[r])
        dxn, dg2 = rmsnorm_backward(x1[r], w.g2, eps, dn2)
        dx1.append(dr[r] + dxn)
        parts.append(SimpleNamespace(w1=dw1, w3=dw3, w2=dw2, g2=dg2, wo=a[r].T @ dx1[r]))
    # attention half: each rank's queries give dK/dV for every position
    dk_part = np.zeros((D, S, hk), F64)
    dv_part = np.zeros((D, S, hk), F64)
    dq = []
    for r in range(D):
        da = dx1[r] @ wo.T
        dqr = np.empty((pos[r].size, h), F64)
        for t in range(n_heads):
            c = slice(t * d, (t + 1) * d)
            kc = slice((t // grp) * d, (t // grp + 1) * d)
            gq, gk, gv = causal_attention_backward(q[r][:, c], pos[r], k_full[:, kc],
                                                   v_full[:, kc], da[:, c])
            dqr[:, c] = rope(gq, -pos[r], rope_theta)
            dk_part[r][:, kc] += gk
            dv_part[r][:, kc] += gv
        dq.append(dqr)
    # reduce-scatter: the owner of each position sums every rank's contribution
    dk_sum, dv_sum = dk_part.sum(axis=0), dv_part.sum(axis=0)
    dx = []
    for r in range(D):
        dk_own = rope_heads(dk_sum[pos[r]], -pos[r], d, rope_theta)
        dv_own = dv_sum[pos[r]]
        dn1 = dq[r] @ wq.T + dk_own @ wk.T + dv_own @ wv.T
        dxn, dg1 = rmsnorm_backward(xr[r], w.g1, eps, dn1)
        dx.append(dx1[r] + dxn)
        p = parts[r]
        p.g1, p.wq, p.wk, p.wv = dg1, n1[r].T @ dq[r], n1[r].T @ dk_own, n1[r].T @ dv_own
    return dx, parts


def rope_heads(m, p, d, theta):
    """rope() applied to every d-column head of m."""
    return np.concatenate([rope(m[:, t * d:(t + 1) * d], p, theta) for t in range(m.shape[1] // d)],
                          axis=1)


def sum_partials(parts):
    """Full weight gradients as the sum of the ranks' partials (what the
    reduce-scatter to each shard's owner computes)."""
    keys = ("g1", "wq", "wk", "wv", "wo", "g2", "w1", "w3", "w2")
    return SimpleNamespace(**{k: sum(getattr(p, k) for p in parts) for k in keys})


__all__ = ["rmsnorm_backward", "swiglu_backward", "causal_attention_backward", "layer_backward",
           "fold_schedule_backward", "sum_partials", "unzigzag"]
