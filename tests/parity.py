"""The parity bar between the HIP path and the oracle (pure numpy; used by
the GPU tests and pinned on the CPU by test_parity_check.py).

Whole tensor: relative Frobenius error <= tol (1e-2 for bf16 workloads,
1e-4 for fp32).  Block delta (x1 - x, out - x1): its error, beyond the
output's own storage rounding, <= tol of the delta's norm.

Local: the same two bounds for every (row, block of `block` columns) with
2 * tol in place of tol.  Why 2 * tol: a correct result's error comes from
per-element roundings -- bf16 storage of the normalised input, Q, K, V, the
probabilities, the per-shard attention output and the SwiGLU product, each
at most u = 2^-9 relative (fp32: 2^-24) -- spread over every row and column,
so each 128-element block carries about the global relative error (2-6e-3
measured on the bf16 workloads: sqrt(6) u = 4.8e-3 is the norm-wise size of
six independent roundings), give or take the sampling spread of 128
squared errors (about 8%).  A localized defect (one head of one query tile,
one split segment merged wrongly) puts all its error into the blocks of the
rows it touches: a 20% error in one head of one tile moves that tile's rows
by 0.2 / sqrt(H) ~ 3.5e-2 of their attention delta (H = 32), twice the local
bar, while moving the global norm by 0.2 / sqrt(32 * 64) ~ 4e-3, under the
global one.  Where the residual stream dominates (x ~ N(0, 1) at the 7B shape
the attention delta is ~0.04 per element), the delta's bar is mostly the bf16
rounding of x1 (~5% of the delta), so the low-residual workloads (x ~
N(0, 0.02^2), same shapes) are the ones that hold attention to the local bar.
"""
import numpy as np

import synth


def tol(cfg) -> float:
    """Relative Frobenius bound: 1e-2 for bf16 storage, 1e-4 for fp32."""
    return 1e-2 if cfg.dtype == "bf16" else 1e-4


def rel_fro(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / (n if n > 0 else 1.0))


def storage_round(cfg, a):
    """The oracle value as the output dtype would store it."""
    a = np.asarray(a, np.float64)
    r = synth.bf16_round(a.astype(np.float32)) if cfg.dtype == "bf16" else a.astype(np.float32)
    return r.astype(np.float64)


def _blocks(a, block):
    """Per (row, column block) Frobenius norms of a 2-D array."""
    a = np.asarray(a, np.float64)
    rows, cols = a.shape
    nb = -(-cols // block)
    pad = np.zeros((rows, nb * block))
    pad[:, :cols] = a
    return np.sqrt((pad.reshape(rows, nb, block) ** 2).sum(axis=2))


def compare(cfg, got, want, base=None, want_base=None, block=None):
    """The parity verdict: (ok, message, stats).  block = columns per local
    block (the head dim by default)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if got.ndim == 1:
        got, want = got[None, :], want[None, :]
        base = None if base is None else np.asarray(base, np.float64)[None, :]
        want_base = None if want_base is None else np.asarray(want_base, np.float64)[None, :]
    blk = block or cfg.head_dim
    t = tol(cfg)
    e = rel_fro(got, want)
    ok = bool(e <= t) and bool(np.all(np.isfinite(got)))
    msg = f"rel {e:.3e}"
    # local bound on the output itself
    rnd_out = _blocks(want - storage_round(cfg, want), blk)
    err_b = _blocks(got - want, blk)
    ref_b = _blocks(want, blk)
    bound_b = 2 * t * ref_b + 1.25 * rnd_out
    worst = float(np.max(err_b / np.maximum(ref_b, 1e-300)))
    ok_b = bool(np.all(err_b <= bound_b))
    stats = {"rel": e, "block_rel_max": worst, "block_ok": ok_b}
    msg += f", worst block {worst:.3e}"
    if base is not None:
        base = np.asarray(base, np.float64)
        want_base = np.asarray(want_base, np.float64)
        dref = want - want_base
        derr = (got - base) - dref
        err = np.linalg.norm(derr)
        rnd = np.linalg.norm(want - storage_round(cfg, want))
        rnd_b = rnd_out.copy()
        if want_base is not base:
            rnd += np.linalg.norm(want_base - storage_round(cfg, want_base))
            rnd_b = rnd_b + _blocks(want_base - storage_round(cfg, want_base), blk)
        dn = max(np.linalg.norm(dref), 1e-300)
        bound = t * np.linalg.norm(dref) + 1.25 * rnd
        ok = ok and bool(err <= bound)
        db = _blocks(dref, blk)
        de = _blocks(derr, blk)
        dbound = 2 * t * db + 1.25 * rnd_b
        ok_db = bool(np.all(de <= dbound))
        # worst block of the delta, beyond its rounding allowance, in units of the local bar
        excess = float(np.max(de / np.maximum(dbound, 1e-300)))
        stats.update(delta_rel=err / dn, delta_block_ok=ok_db, delta_block_worst_of_bar=excess)
        msg += (f", delta err {err / dn:.3e} of |delta| (bound {bound / dn:.3e}, "
                f"storage rounding {rnd / dn:.3e}), worst delta block {excess:.2f} of its bar")
        ok_b = ok_b and ok_db
    if not ok_b:
        r, c = np.unravel_index(np.argmax(err_b / np.maximum(bound_b, 1e-300)), err_b.shape)
        msg += f"; local bound broken (e.g. row {r}, columns {c * blk}..{c * blk + blk - 1})"
    return ok and ok_b, msg, stats
