"""Thin ctypes binding of libtsp.so (C ABI in include/tsp.h).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch supplies device memory and streams.  The helpers at the bottom put
weights into the packed shard layout the ABI defines (tensor slicing and
transposes on the device) and size the gathered K/V buffer.

If libtsp.so is missing this module raises on first use; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtsp.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "tsp.h")

TSP_BF16, TSP_F32 = 0, 1
TSP_WS_ATTN, TSP_WS_MLP, TSP_WS_LAYER, TSP_WS_KV, TSP_WS_MLP_BWD, TSP_WS_ATTN_BWD = 1, 2, 3, 4, 5, 6
TSP_WS_LAYER_BWD, TSP_WS_LAYER_BWD_FINISH = 7, 8
TSP_F_DELAY_COPY, TSP_F_POISON_SLOTS, TSP_F_NO_OVERLAP, TSP_F_PROFILE = 1, 2, 4, 8
TSP_F_RESCALE_TEST = 16
TSP_F_KV_STREAM = 32
TSP_F_SHARD_LAUNCH = 64
KERNELS = ["rmsnorm", "qkv", "attn", "merge", "oproj", "w13", "w2"]  # TSP_K_* order
STATUS = {0: "TSP_OK", -1: "TSP_E_INVAL", -2: "TSP_E_SHAPE", -3: "TSP_E_ALIGN",
          -4: "TSP_E_WORKSPACE", -5: "TSP_E_DTYPE", -6: "TSP_E_HIP"}


class TspError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class TspDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("fold", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("seq", ctypes.c_int64), ("eps", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("rope_theta", ctypes.c_float)]


_lib = None
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_pp = ctypes.POINTER(ctypes.c_void_p)


def lib() -> ctypes.CDLL:
    """Load libtsp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m folded_tensor_sequence_rank_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        D = ctypes.POINTER(TspDims)
        L.tsp_workspace_bytes.argtypes = [D, ctypes.c_int]
        L.tsp_workspace_bytes.restype = _sz
        L.tsp_strerror.argtypes = [ctypes.c_int]
        L.tsp_strerror.restype = ctypes.c_char_p
        L.tsp_last_error.argtypes = []
        L.tsp_last_error.restype = ctypes.c_char_p
        L.tsp_zigzag_positions.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(ctypes.c_int64)]
        L.tsp_attn_shard.argtypes = [D, _vp, _vp, _pp, _vp, _vp, _vp, _sz, _vp, _vp]
        L.tsp_attn_shard_save.argtypes = [D, _vp, _vp, _pp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp]
        L.tsp_mlp_shard.argtypes = [D, _vp, _vp, _pp, _vp, _vp, _sz, _vp, _vp]
        L.tsp_layer_shard.argtypes = [D, _vp, _vp, _pp, _vp, _vp, _pp, _vp, _vp, _sz, _vp, _vp]
        L.tsp_kv_shard.argtypes = [D, _vp, _vp, _pp, _vp, _vp, _sz, _vp]
        L.tsp_layer_shard_noalloc.argtypes = [D, _vp, _vp, _pp, _vp, _vp, _pp, _vp, _vp, _vp]
        L.tsp_mlp_shard_backward.argtypes = [D, _vp, _vp, _pp, _vp, _vp, _vp, _pp, _vp, _sz, _vp]
        L.tsp_attn_core_backward.argtypes = [D, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        L.tsp_layer_shard_backward.argtypes = [D, _vp, _vp, _vp, _pp, _vp, _vp, _pp, _vp, _vp, _vp, _vp,
                                               _vp, _pp, _pp, _vp, _vp, _vp, _sz, _vp]
        L.tsp_kv_grad_reduce.argtypes = [D, _pp, _vp, _vp]
        L.tsp_layer_shard_backward_finish.argtypes = [D, _vp, _vp, _pp, _vp, _vp, _vp, _vp, _vp, _pp, _vp,
                                                      _sz, _vp]
        L.tsp_clock_probe.argtypes = [_vp, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int32), _vp]
        L.tsp_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
        for f in ("tsp_attn_shard", "tsp_attn_shard_save", "tsp_mlp_shard", "tsp_layer_shard", "tsp_kv_shard",
                  "tsp_mlp_shard_backward", "tsp_attn_core_backward", "tsp_layer_shard_backward",
                  "tsp_kv_grad_reduce", "tsp_layer_shard_backward_finish",
                  "tsp_zigzag_positions", "tsp_profile_read", "tsp_clock_probe",
                  "tsp_layer_shard_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def header_symbols() -> List[str]:
    """Function names declared in include/tsp.h."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tsp_[a-z_]+)\s*\(", src)))


def make_dims(cfg, rank: int, flags: int = 0, seq: Optional[int] = None) -> TspDims:
    """TspDims from any object with hidden, n_heads, head_dim, ffn, fold, seq,
    eps and dtype ("bf16" or "f32") attributes, and optionally batch (the
    micro-batch of sequences, default 1), n_kv_heads (default n_heads) and
    rope_theta (default 0: no rotary embedding)."""
    return TspDims(cfg.hidden, cfg.n_heads, cfg.head_dim, cfg.ffn, cfg.fold, rank,
                   cfg.seq if seq is None else seq, cfg.eps,
                   TSP_BF16 if cfg.dtype == "bf16" else TSP_F32, flags,
                   int(getattr(cfg, "batch", 1)), int(getattr(cfg, "n_kv_heads", 0) or 0),
                   float(getattr(cfg, "rope_theta", 0.0) or 0.0))


def _check(rc: int):
    if rc != 0:
        raise TspError(rc, lib().tsp_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _ptrs(ts: Sequence) -> ctypes.Array:
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t)
    return arr


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_sizes(dims: TspDims, which: int, **bufs):
    """Byte sizes of the tensors passed for one call against what the dims
    make the library read or write (the C ABI takes plain pointers and
    cannot check them).  Integer addresses are not checked, nor are calls
    whose dims the library rejects (it reports those itself)."""
    if workspace_bytes(dims, which) == 0:
        return
    es = 2 if dims.dtype == TSP_BF16 else 4
    h, D, d = dims.hidden, dims.fold, dims.head_dim
    B = max(dims.batch, 1)
    rows = B * (dims.seq // D)
    hs = h // D
    ks = (dims.n_kv_heads or dims.n_heads) * d // D
    need = {"x": rows * h, "x1": rows * h, "out": rows * h, "g1": h, "g2": h,
            "kv": 2 * (dims.n_kv_heads or dims.n_heads) * B * dims.seq * d,
            "w_attn": (hs + 2 * ks) * h + h * hs, "w_mlp": 3 * (dims.ffn // D) * h}
    for name, t in bufs.items():
        ts = t if name in ("w_attn", "w_mlp") else [t]
        if name in ("w_attn", "w_mlp") and len(ts) != D:
            raise ValueError(f"{name}: {len(ts)} shards for fold {D}")
        for i, u in enumerate(ts):
            if hasattr(u, "numel") and _nbytes(u) < need[name] * es:
                raise ValueError(f"{name}{'' if len(ts) == 1 else f'[{i}]'}: {_nbytes(u)} bytes, "
                                 f"the dims need {need[name] * es}")


def workspace_bytes(dims: TspDims, which: int) -> int:
    return int(lib().tsp_workspace_bytes(ctypes.byref(dims), which))


def zigzag_positions(seq: int, fold: int, rank: int) -> np.ndarray:
    out = np.zeros(max(seq // fold, 1), np.int64)
    _check(lib().tsp_zigzag_positions(seq, fold, rank,
                                      out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
    return out[: seq // fold]


def tsp_attn_shard(dims, x, g1, w_attn, kv, x1, ws, stream=None, copy_stream=None):
    _check_sizes(dims, TSP_WS_ATTN, x=x, g1=g1, w_attn=w_attn, kv=kv, x1=x1)
    _check(lib().tsp_attn_shard(ctypes.byref(dims), _ptr(x), _ptr(g1), _ptrs(w_attn), _ptr(kv),
                                _ptr(x1), _ptr(ws), _nbytes(ws), _stream(stream),
                                None if copy_stream is None else _stream(copy_stream)))


def _saved_sizes(dims):
    """Bytes of tsp_attn_shard_save's attn_out and lse."""
    es = 2 if dims.dtype == TSP_BF16 else 4
    BT = max(dims.batch, 1) * (dims.seq // dims.fold)
    return BT * dims.hidden * es, dims.n_heads * BT * 4


def tsp_attn_shard_save(dims, x, g1, w_attn, kv, x1, attn_out, lse, ws, stream=None, copy_stream=None):
    """tsp_attn_shard that also keeps each head group's attention output
    attn_out [B*T][h] and the rows' log2 softmax normalisers lse [H][B*T]
    (fp32) for tsp_layer_shard_backward (include/tsp.h)."""
    _check_sizes(dims, TSP_WS_ATTN, x=x, g1=g1, w_attn=w_attn, kv=kv, x1=x1)
    na, nl = _saved_sizes(dims)
    _need("attn_out", attn_out, na)
    _need("lse", lse, nl)
    _check(lib().tsp_attn_shard_save(ctypes.byref(dims), _ptr(x), _ptr(g1), _ptrs(w_attn), _ptr(kv),
                                     _ptr(x1), _ptr(attn_out), _ptr(lse), _ptr(ws), _nbytes(ws),
                                     _stream(stream), None if copy_stream is None else _stream(copy_stream)))


def tsp_mlp_shard(dims, x1, g2, w_mlp, out, ws, stream=None, copy_stream=None):
    _check_sizes(dims, TSP_WS_MLP, x1=x1, g2=g2, w_mlp=w_mlp, out=out)
    _check(lib().tsp_mlp_shard(ctypes.byref(dims), _ptr(x1), _ptr(g2), _ptrs(w_mlp), _ptr(out),
                               _ptr(ws), _nbytes(ws), _stream(stream),
                               None if copy_stream is None else _stream(copy_stream)))


def tsp_layer_shard(dims, x, g1, w_attn, kv, g2, w_mlp, out, ws, stream=None, copy_stream=None):
    _check_sizes(dims, TSP_WS_LAYER, x=x, g1=g1, w_attn=w_attn, kv=kv, g2=g2, w_mlp=w_mlp, out=out)
    _check(lib().tsp_layer_shard(ctypes.byref(dims), _ptr(x), _ptr(g1), _ptrs(w_attn), _ptr(kv),
                                 _ptr(g2), _ptrs(w_mlp), _ptr(out), _ptr(ws), _nbytes(ws),
                                 _stream(stream),
                                 None if copy_stream is None else _stream(copy_stream)))


def tsp_layer_shard_noalloc(dims, x, g1, w_attn, kv, g2, w_mlp, out, stream=None, copy_stream=None):
    """tsp_layer_shard on the library's static scratch (include/tsp.h): no
    workspace argument, no allocation."""
    _check_sizes(dims, TSP_WS_LAYER, x=x, g1=g1, w_attn=w_attn, kv=kv, g2=g2, w_mlp=w_mlp, out=out)
    _check(lib().tsp_layer_shard_noalloc(ctypes.byref(dims), _ptr(x), _ptr(g1), _ptrs(w_attn), _ptr(kv),
                                         _ptr(g2), _ptrs(w_mlp), _ptr(out), _stream(stream),
                                         None if copy_stream is None else _stream(copy_stream)))


NOALLOC_SCRATCH_BYTES = 256 << 20


def tsp_kv_shard(dims, x, g1, w_attn, kv, ws, stream=None):
    _check_sizes(dims, TSP_WS_KV, x=x, g1=g1, w_attn=w_attn, kv=kv)
    _check(lib().tsp_kv_shard(ctypes.byref(dims), _ptr(x), _ptr(g1), _ptrs(w_attn), _ptr(kv),
                              _ptr(ws), _nbytes(ws), _stream(stream)))


def tsp_mlp_shard_backward(dims, x1, g2, w_mlp, dout, dx1, dg2, dw_mlp, ws, stream=None):
    """Backward of the MLP half (include/tsp.h): dx1 in the dims' dtype, and
    this rank's partial gradients dg2 [h] and dw_mlp (D fp32 tensors of
    3*Fs*h elements in the packed shard layout)."""
    _check_sizes(dims, TSP_WS_MLP_BWD, x1=x1, g2=g2, w_mlp=w_mlp, out=dout)
    _check_sizes(dims, TSP_WS_MLP_BWD, x=dx1)
    D, h = dims.fold, dims.hidden
    if hasattr(dg2, "numel") and _nbytes(dg2) < 4 * h:
        raise ValueError(f"dg2: {_nbytes(dg2)} bytes, the dims need {4 * h}")
    need = 4 * 3 * (dims.ffn // D) * h
    if len(dw_mlp) != D:
        raise ValueError(f"dw_mlp: {len(dw_mlp)} shards for fold {D}")
    for i, t in enumerate(dw_mlp):
        if hasattr(t, "numel") and _nbytes(t) < need:
            raise ValueError(f"dw_mlp[{i}]: {_nbytes(t)} bytes, the dims need {need}")
    _check(lib().tsp_mlp_shard_backward(ctypes.byref(dims), _ptr(x1), _ptr(g2), _ptrs(w_mlp),
                                        _ptr(dout), _ptr(dx1), _ptr(dg2), _ptrs(dw_mlp), _ptr(ws),
                                        _nbytes(ws), _stream(stream)))


def tsp_attn_core_backward(dims, q, kv, dout, dq, dk, dv, ws, stream=None):
    """Backward of the attention core for one shard's head group
    (include/tsp.h): dq [Hd][B*T][d], and this rank's partial dk, dv
    [Hkd][B*S][d], all fp32."""
    D, d = dims.fold, dims.head_dim
    B = max(dims.batch, 1)
    T = dims.seq // D
    Hd = dims.n_heads // D
    Hkd = (dims.n_kv_heads or dims.n_heads) // D
    es = 2 if dims.dtype == TSP_BF16 else 4
    need = {"q": Hd * B * T * d * es, "kv": 2 * Hkd * B * dims.seq * d * es,
            "dout": B * T * Hd * d * es, "dq": Hd * B * T * d * 4, "dk": Hkd * B * dims.seq * d * 4,
            "dv": Hkd * B * dims.seq * d * 4}
    for name, t in (("q", q), ("kv", kv), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if hasattr(t, "numel") and _nbytes(t) < need[name]:
            raise ValueError(f"{name}: {_nbytes(t)} bytes, the dims need {need[name]}")
    _check(lib().tsp_attn_core_backward(ctypes.byref(dims), _ptr(q), _ptr(kv), _ptr(dout), _ptr(dq),
                                        _ptr(dk), _ptr(dv), _ptr(ws), _nbytes(ws), _stream(stream)))


def _need(name, t, nbytes):
    if hasattr(t, "numel") and _nbytes(t) < nbytes:
        raise ValueError(f"{name}: {_nbytes(t)} bytes, the dims need {nbytes}")


def _bwd_sizes(dims):
    D, d, h = dims.fold, dims.head_dim, dims.hidden
    B = max(dims.batch, 1)
    H, Hkv = dims.n_heads, dims.n_kv_heads or dims.n_heads
    BT, BS = B * (dims.seq // D), B * dims.seq
    hs, ks = h // D, Hkv * d // D
    return {"dq": H * BT * d * 4, "dkv": 2 * Hkv * BS * d * 4, "dkv_own": 2 * Hkv * BT * d * 4,
            "dw_o": h * hs * 4, "dw_qkv": (hs + 2 * ks) * h * 4, "dw_mlp": 3 * (dims.ffn // D) * h * 4,
            "gain": h * 4}


def tsp_layer_shard_backward(dims, x, x1, g1, w_attn, kv, g2, w_mlp, dout, dx1, dg2, dw_mlp, dw_o, dq, dkv,
                             ws, stream=None, attn_saved=None, lse_saved=None):
    """Part 1 of the whole layer's backward (include/tsp.h): dx1, the partial
    dg2, dw_mlp and dw_o, the unrotated dq [H][B*T][d] and the partial dkv
    [D][2][Hkv/D][B*S][d] (fp32).  attn_saved / lse_saved: the attn_out and
    lse of tsp_attn_shard_save (the forward attention is then not
    recomputed), or both None."""
    _check_sizes(dims, TSP_WS_LAYER_BWD, x=x, g1=g1, w_attn=w_attn, kv=kv, g2=g2, w_mlp=w_mlp, out=dout)
    _check_sizes(dims, TSP_WS_LAYER_BWD, x1=x1)
    _check_sizes(dims, TSP_WS_LAYER_BWD, x=dx1)
    n = _bwd_sizes(dims)
    for name, t in (("dq", dq), ("dkv", dkv), ("dg2", dg2)):
        _need(name, t, n[name] if name != "dg2" else n["gain"])
    na, nl = _saved_sizes(dims)
    _need("attn_saved", attn_saved, na)
    _need("lse_saved", lse_saved, nl)
    for name, ts in (("dw_mlp", dw_mlp), ("dw_o", dw_o)):
        if len(ts) != dims.fold:
            raise ValueError(f"{name}: {len(ts)} shards for fold {dims.fold}")
        for i, t in enumerate(ts):
            _need(f"{name}[{i}]", t, n[name])
    _check(lib().tsp_layer_shard_backward(ctypes.byref(dims), _ptr(x), _ptr(x1), _ptr(g1), _ptrs(w_attn),
                                          _ptr(kv), _ptr(g2), _ptrs(w_mlp), _ptr(dout),
                                          _ptr(attn_saved), _ptr(lse_saved), _ptr(dx1), _ptr(dg2),
                                          _ptrs(dw_mlp), _ptrs(dw_o), _ptr(dq), _ptr(dkv), _ptr(ws),
                                          _nbytes(ws), _stream(stream)))


def tsp_kv_grad_reduce(dims, dkv_parts, dkv_own, stream=None):
    """The dK/dV exchange's sums for rank dims.rank: dkv_own [D][2][Hkv/D][B*T][d]
    (fp32) from the D ranks' part-1 dkv buffers."""
    n = _bwd_sizes(dims)
    if len(dkv_parts) != dims.fold:
        raise ValueError(f"dkv_parts: {len(dkv_parts)} buffers for fold {dims.fold}")
    for i, t in enumerate(dkv_parts):
        _need(f"dkv_parts[{i}]", t, n["dkv"])
    _need("dkv_own", dkv_own, n["dkv_own"])
    _check(lib().tsp_kv_grad_reduce(ctypes.byref(dims), _ptrs(dkv_parts), _ptr(dkv_own), _stream(stream)))


def tsp_layer_shard_backward_finish(dims, x, g1, w_attn, dx1, dq, dkv_own, dx, dg1, dw_qkv, ws, stream=None):
    """Part 2 of the whole layer's backward (include/tsp.h): dx, the partial
    dg1 and dw_qkv (fp32, packed Q|K|V block layout)."""
    _check_sizes(dims, TSP_WS_LAYER_BWD_FINISH, x=x, g1=g1, w_attn=w_attn)
    _check_sizes(dims, TSP_WS_LAYER_BWD_FINISH, x1=dx1, out=dx)
    n = _bwd_sizes(dims)
    _need("dq", dq, n["dq"])
    _need("dkv_own", dkv_own, n["dkv_own"])
    _need("dg1", dg1, n["gain"])
    if len(dw_qkv) != dims.fold:
        raise ValueError(f"dw_qkv: {len(dw_qkv)} shards for fold {dims.fold}")
    for i, t in enumerate(dw_qkv):
        _need(f"dw_qkv[{i}]", t, n["dw_qkv"])
    _check(lib().tsp_layer_shard_backward_finish(ctypes.byref(dims), _ptr(x), _ptr(g1), _ptrs(w_attn),
                                                 _ptr(dx1), _ptr(dq), _ptr(dkv_own), _ptr(dx), _ptr(dg1),
                                                 _ptrs(dw_qkv), _ptr(ws), _nbytes(ws), _stream(stream)))


def tsp_profile_read(reset: bool = True) -> dict:
    """Per-kernel-class totals of calls made with TSP_F_PROFILE:
    {name: (total_ms, launches)}."""
    ms = (ctypes.c_double * len(KERNELS))()
    n = (ctypes.c_int64 * len(KERNELS))()
    _check(lib().tsp_profile_read(ms, n, 1 if reset else 0))
    return {k: (ms[i], n[i]) for i, k in enumerate(KERNELS)}


def tsp_clock_probe(samples, n: int, interval_us: int, stream=None) -> int:
    """Enqueue the clock probe (include/tsp.h) writing n (wall tick, shader
    cycle) pairs into `samples` (an int64 device tensor of >= 2n elements);
    returns the wall clock's rate in kHz."""
    if hasattr(samples, "numel") and _nbytes(samples) < 16 * n:
        raise ValueError(f"samples: {_nbytes(samples)} bytes, {n} samples need {16 * n}")
    khz = ctypes.c_int32(0)
    _check(lib().tsp_clock_probe(_ptr(samples), n, interval_us, ctypes.byref(khz), _stream(stream)))
    return int(khz.value)


def clock_mhz(samples: np.ndarray, wall_khz: int) -> np.ndarray:
    """Effective clock (MHz) over each interval between consecutive probe
    samples: shader cycles / wall ticks * wall-clock rate."""
    s = np.asarray(samples, np.int64).reshape(-1, 2).astype(np.float64)
    dt = np.diff(s[:, 0])
    dc = np.diff(s[:, 1])
    ok = dt > 0
    return dc[ok] / dt[ok] * (wall_khz / 1000.0)


# ----------------------------------------------------------------------------
# Layout helpers (device tensors in, device tensors out)
# ----------------------------------------------------------------------------

def pack_attn_shards(wq, wk, wv, wo, fold: int):
    """Packed attention shards from math-layout weights (Q = n @ wq; wq, wo
    [h, h]; wk, wv [h, Hkv*d]): per shard j the output-major blocks of the
    W_Q columns of head group j and of the W_K, W_V columns of K/V head group
    j, then the output-major block of W_O's rows of head group j."""
    import torch
    h = wq.shape[0]
    hs = h // fold
    ks = wk.shape[1] // fold
    out = []
    for j in range(fold):
        c = slice(j * hs, (j + 1) * hs)
        k = slice(j * ks, (j + 1) * ks)
        out.append(torch.cat([wq[:, c].t().reshape(-1), wk[:, k].t().reshape(-1),
                              wv[:, k].t().reshape(-1), wo[c, :].t().reshape(-1)]).contiguous())
    return out


def pack_mlp_shards(w1, w3, w2, fold: int):
    """Packed MLP shards from math-layout weights (w1, w3 [h, F]; w2 [F, h])."""
    import torch
    F = w1.shape[1]
    fs = F // fold
    out = []
    for j in range(fold):
        c = slice(j * fs, (j + 1) * fs)
        out.append(torch.cat([w1[:, c].t().reshape(-1), w3[:, c].t().reshape(-1),
                              w2[c, :].t().reshape(-1)]).contiguous())
    return out


def kv_elems(cfg) -> int:
    """Elements of the gathered K/V buffer: D blocks of 2 * (Hkv/D) * B * S * d."""
    hkv = int(getattr(cfg, "n_kv_heads", 0) or cfg.n_heads)
    return 2 * hkv * cfg.seq * cfg.head_dim * int(getattr(cfg, "batch", 1))
