"""Host-side checks of the C ABI: the library loads, exports every function
include/tsp.h declares, sizes workspaces, and rejects bad arguments with the
documented status before touching a GPU."""
import ctypes

import numpy as np
import pytest

import oracle.tsp_oracle as O
import synth
from folded_tensor_sequence_rank_amd import tsp

C3 = synth.get_config("7b_s64k")
TINY = synth.get_config("tiny_fp32")


def test_exports_every_declared_symbol():
    L = tsp.lib()
    syms = tsp.header_symbols()
    assert {"tsp_attn_shard", "tsp_mlp_shard", "tsp_layer_shard", "tsp_kv_shard",
            "tsp_workspace_bytes", "tsp_strerror", "tsp_last_error",
            "tsp_zigzag_positions"} <= set(syms)
    for s in syms:
        assert hasattr(L, s), s


def test_strerror():
    L = tsp.lib()
    for code, name in tsp.STATUS.items():
        assert L.tsp_strerror(code).decode()
    assert L.tsp_strerror(12345).decode() == "unknown status"


def test_zigzag_helper_matches_statement_and_oracle():
    # The tiny workload's rank 1 of 4 holds chunks 1 and 6 of 32 tokens.
    p = tsp.zigzag_positions(256, 4, 1)
    assert np.array_equal(p, np.r_[32:64, 192:224])
    for S, D in [(16, 1), (64, 2), (1024, 8), (96, 3)]:
        for r in range(D):
            assert np.array_equal(tsp.zigzag_positions(S, D, r), O.zigzag_positions(S, D, r))
    with pytest.raises(tsp.TspError) as e:
        tsp.zigzag_positions(100, 8, 0)
    assert e.value.name == "TSP_E_SHAPE"


def test_workspace_sizes():
    d = tsp.make_dims(C3, 3)
    a = tsp.workspace_bytes(d, tsp.TSP_WS_ATTN)
    m = tsp.workspace_bytes(d, tsp.TSP_WS_MLP)
    l = tsp.workspace_bytes(d, tsp.TSP_WS_LAYER)
    k = tsp.workspace_bytes(d, tsp.TSP_WS_KV)
    T, h = 8192, 4096
    assert a > 2 * 2 * 4 * 65536 * 128 * 2      # two K/V slots of one head group
    assert l >= a + m + T * h * 2                 # x1 kept between the halves
    assert k >= T * h * 2
    assert l < 2 << 30                            # about 1 GB at the 64K workload
    bad = tsp.make_dims(C3.with_(fold=3), 0)
    assert tsp.workspace_bytes(bad, tsp.TSP_WS_ATTN) == 0
    assert tsp.workspace_bytes(d, 99) == 0


def _call_attn(dims, x=16, g=16, w=None, kv=16, out=16, ws=16, ws_bytes=1 << 40):
    """Call tsp_attn_shard with fake (never dereferenced) addresses."""
    L = tsp.lib()
    D = dims.fold if dims.fold > 0 else 1
    arr = (ctypes.c_void_p * D)(*([w if w is not None else 4096] * D))
    return L.tsp_attn_shard(ctypes.byref(dims), x, g, arr, kv, out, ws, ws_bytes, None, None)


@pytest.mark.parametrize("case,field,value,status", [
    ("rank_high", "rank", 8, "TSP_E_INVAL"),
    ("rank_neg", "rank", -1, "TSP_E_INVAL"),
    ("fold_zero", "fold", 0, "TSP_E_INVAL"),
    ("dtype", "dtype", 7, "TSP_E_DTYPE"),
    ("h_ne_Hd", "hidden", 4000, "TSP_E_SHAPE"),
    ("head_dim", "head_dim", 96, "TSP_E_SHAPE"),
    ("seq_2D", "seq", 65536 + 8, "TSP_E_SHAPE"),
    ("ffn_D", "ffn", 11001, "TSP_E_SHAPE"),
    ("batch_neg", "batch", -2, "TSP_E_INVAL"),
    ("batch_positions", "batch", 1 << 15, "TSP_E_SHAPE"),   # B*S past 2^31 - 1
    ("kv_heads_neg", "n_kv_heads", -8, "TSP_E_INVAL"),
    ("kv_heads_divide_H", "n_kv_heads", 24, "TSP_E_SHAPE"),   # 32 % 24
    ("kv_heads_fold", "n_kv_heads", 4, "TSP_E_SHAPE"),        # 4 K/V heads over 8 ranks
    ("rope_neg", "rope_theta", -1.0, "TSP_E_INVAL"),
    ("rope_nan", "rope_theta", float("nan"), "TSP_E_INVAL"),
    ("rope_inf", "rope_theta", float("inf"), "TSP_E_INVAL"),
    ("rope_below_one", "rope_theta", 0.5, "TSP_E_INVAL"),
])
def test_bad_dims(case, field, value, status):
    d = tsp.make_dims(C3, 3)
    if field == "head_dim":
        d.head_dim, d.n_heads = 96, 4096 // 96  # keeps nothing consistent on purpose
    else:
        setattr(d, field, value)
    rc = _call_attn(d)
    assert tsp.STATUS[rc] == status, (rc, tsp.lib().tsp_last_error())


def test_bad_pointers_and_workspace():
    d = tsp.make_dims(C3, 3)
    assert tsp.STATUS[_call_attn(d, x=0)] == "TSP_E_INVAL"
    assert tsp.STATUS[_call_attn(d, w=0)] == "TSP_E_INVAL"
    assert tsp.STATUS[_call_attn(d, kv=24)] == "TSP_E_ALIGN"
    assert tsp.STATUS[_call_attn(d, w=4100)] == "TSP_E_ALIGN"
    assert tsp.STATUS[_call_attn(d, ws_bytes=1000)] == "TSP_E_WORKSPACE"
    assert "workspace" in tsp.lib().tsp_last_error().decode()
    # null host pointer array
    rc = tsp.lib().tsp_attn_shard(ctypes.byref(d), 16, 16, None, 16, 16, 16, 1 << 40, None, None)
    assert tsp.STATUS[rc] == "TSP_E_INVAL"


def test_empty_sequence_is_a_no_op():
    d = tsp.make_dims(C3, 3, seq=0)
    assert _call_attn(d, x=0, kv=0, out=0, ws=0, ws_bytes=0) == 0
    L = tsp.lib()
    arr = (ctypes.c_void_p * 8)()
    assert L.tsp_mlp_shard(ctypes.byref(d), None, None, arr, None, None, 0, None, None) == 0
    assert L.tsp_kv_shard(ctypes.byref(d), None, None, arr, None, None, 0, None) == 0


def test_dims_struct_layout():
    assert ctypes.sizeof(tsp.TspDims) == 56
    assert tsp.TspDims.seq.offset == 24 and tsp.TspDims.flags.offset == 40
    assert tsp.TspDims.batch.offset == 44
    assert tsp.TspDims.n_kv_heads.offset == 48 and tsp.TspDims.rope_theta.offset == 52


def test_gqa_rope_dims_and_workspace():
    """n_kv_heads 0 means H; grouped K/V shrink the K/V slots and the gathered
    buffer by H/Hkv; the rotary embedding needs no memory."""
    mha = tsp.make_dims(C3, 3)
    same = tsp.make_dims(C3.with_(n_kv_heads=32, rope_theta=10000.0), 3)
    gqa = tsp.make_dims(C3.with_(n_kv_heads=8), 3)
    for dm in (mha, same, gqa):  # one shard per launch, so the slots hold one shard each
        dm.flags |= tsp.TSP_F_SHARD_LAUNCH
    assert mha.n_kv_heads == 0 and same.n_kv_heads == 32 and abs(same.rope_theta - 1e4) < 1e-3
    for which in (tsp.TSP_WS_ATTN, tsp.TSP_WS_MLP, tsp.TSP_WS_LAYER, tsp.TSP_WS_KV):
        assert tsp.workspace_bytes(same, which) == tsp.workspace_bytes(mha, which)
    a_mha = tsp.workspace_bytes(mha, tsp.TSP_WS_ATTN)
    a_gqa = tsp.workspace_bytes(gqa, tsp.TSP_WS_ATTN)
    # two K/V slots of 2 * (H/D) * S * d elements shrink to 2 * (Hkv/D) * S * d
    slot = 2 * 4 * 65536 * 128 * 2
    assert a_mha - a_gqa >= 2 * (slot - slot // 4)
    assert tsp.workspace_bytes(gqa, tsp.TSP_WS_MLP) == tsp.workspace_bytes(mha, tsp.TSP_WS_MLP)
    assert tsp.kv_elems(C3.with_(n_kv_heads=8)) * 4 == tsp.kv_elems(C3)


def test_shards_per_launch_workspace():
    """By default the P = min(4, D/2) shards of a launch group share each QKV,
    attention and W1/W3 launch, and one O (W2) projection covers all D shards:
    its group buffers hold all of W_O (W2) and the attention outputs (SwiGLU
    products) of the layer, and no fp32 partial sum exists.
    TSP_F_SHARD_LAUNCH runs one shard per launch with accumulation groups of
    P shards: two group buffers of half the columns, and the fp32 partial sum.
    The attention's split partials differ too (a launch over more heads
    splits less)."""
    def ws(cfg, flags, which):
        d = tsp.make_dims(cfg, 3 % cfg.fold)
        d.flags |= flags
        return tsp.workspace_bytes(d, which)
    h, F, es = 4096, 11008, 2
    for cfg in (C3, C3.with_(seq=16384), C3.with_(seq=16384, fold=4)):
        D, T, S = cfg.fold, cfg.local_tokens, cfg.seq
        P = min(4, D // 2)
        hs, Fs = h // D, F // D
        qkv = 3 * hs * h * es                   # one packed Q|K|V block
        kvslot = 2 * (32 // D) * S * 128 * es   # one shard's K and V^T over the sequence
        launch = (P - 1) * (2 * qkv + 2 * kvslot + T * hs * es)  # more shards in 2 slots each, and in Q
        # accumulation: all D shards' columns in one group, against two groups of P shards' columns
        # (D = 2P) and the [T][h] fp32 partial sum
        acc_o = (T * h * es + h * h * es) - (T * P * hs * es + 2 * h * P * hs * es + 4 * T * h)
        acc_m = (T * F * es + h * F * es) - (T * P * Fs * es + 2 * h * P * Fs * es + 4 * T * h)
        diff = ws(cfg, 0, tsp.TSP_WS_ATTN) - ws(cfg, tsp.TSP_F_SHARD_LAUNCH, tsp.TSP_WS_ATTN)
        want = launch + acc_o
        assert want - 128 * 2**20 <= diff <= want + 32 * 2**20, (D, S, diff, want)  # split partials
        mlp = ws(cfg, 0, tsp.TSP_WS_MLP) - ws(cfg, tsp.TSP_F_SHARD_LAUNCH, tsp.TSP_WS_MLP)
        want_m = (P - 1) * 2 * 2 * Fs * h * es + acc_m
        assert abs(mlp - want_m) <= 4 * 256, (D, mlp, want_m)  # 256-byte alignment of each buffer


def test_micro_batch_workspace():
    """batch 0 means 1; the activations, K/V slots and attention partials
    grow with the micro-batch while the weight slots do not."""
    one = tsp.make_dims(C3, 3)
    zero = tsp.make_dims(C3, 3)
    zero.batch = 0
    four = tsp.make_dims(C3.with_(batch=4), 3)
    for which in (tsp.TSP_WS_ATTN, tsp.TSP_WS_MLP, tsp.TSP_WS_LAYER, tsp.TSP_WS_KV):
        w1 = tsp.workspace_bytes(one, which)
        assert tsp.workspace_bytes(zero, which) == w1
        w4 = tsp.workspace_bytes(four, which)
        assert w1 < w4 <= 4 * w1 + 4096, (which, w1, w4)
    assert tsp.workspace_bytes(four, tsp.TSP_WS_KV) >= 4 * 8192 * 4096 * 2
    assert tsp.kv_elems(C3.with_(batch=4)) == 4 * tsp.kv_elems(C3)


def test_product_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(tsp, "_lib", None)
    monkeypatch.setattr(tsp, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        tsp.lib()


def test_binding_rejects_undersized_tensors():
    """The binding checks tensor sizes against the dims before any launch (CPU
    tensors stand in: nothing is enqueued when a check fails)."""
    import torch
    cfg = C3.with_(batch=4)
    d = tsp.make_dims(cfg, 3)
    T, h = cfg.local_tokens, cfg.hidden
    one_seq = torch.empty(T * h, dtype=torch.bfloat16)          # one sequence's rows only
    g = torch.empty(h, dtype=torch.bfloat16)
    shards = [torch.empty(4 * 512 * 4096, dtype=torch.bfloat16) for _ in range(8)]
    kv = torch.empty(1, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="x: .* the dims need"):
        tsp.tsp_kv_shard(d, one_seq, g, shards, kv, torch.empty(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="kv"):
        tsp.tsp_kv_shard(d, torch.empty(4 * T * h, dtype=torch.bfloat16), g, shards, kv,
                         torch.empty(256, dtype=torch.uint8))
    with pytest.raises(ValueError, match="shards for fold"):
        tsp.tsp_kv_shard(d, torch.empty(4 * T * h, dtype=torch.bfloat16), g, shards[:7], kv,
                         torch.empty(256, dtype=torch.uint8))


def test_attention_backward_rejects_unsupported_before_gpu():
    """bf16 only, head_dim 64 or 128: rejected from the dims alone."""
    L = tsp.lib()
    for cfg, want in ((TINY, "TSP_E_DTYPE"),
                      (synth.LayerConfig(name="d32", hidden=256, n_heads=8, head_dim=32, ffn=512, seq=512,
                                         fold=2, ranks=(0,), layers=1, dtype="bf16"), "TSP_E_SHAPE")):
        dims = tsp.make_dims(cfg, 0)
        rc = L.tsp_attn_core_backward(ctypes.byref(dims), None, None, None, None, None, None, None, 0, None)
        assert tsp.STATUS[rc] == want, (cfg.name, rc, L.tsp_last_error())


def test_layer_backward_saved_inputs_come_in_pairs():
    """attn_saved without lse_saved (or the reverse) is refused on the host,
    before any pointer is read."""
    L = tsp.lib()
    cfg = synth.LayerConfig(name="b", hidden=256, n_heads=2, head_dim=128, ffn=512, seq=512, fold=2,
                            ranks=(0,), layers=1, dtype="bf16")
    dims = tsp.make_dims(cfg, 0)
    ptrs = (ctypes.c_void_p * 2)(16, 16)
    for a, l in ((16, None), (None, 16)):
        rc = L.tsp_layer_shard_backward(ctypes.byref(dims), 16, 16, 16, ptrs, 16, 16, ptrs, 16, a, l, 16, 16, ptrs,
                                        ptrs, 16, 16, 16, 1 << 40, None)
        assert tsp.STATUS[rc] == "TSP_E_INVAL", (a, l, rc)
        assert "together" in L.tsp_last_error().decode()


@pytest.mark.parametrize("cfg,ok,what", [
    # bf16 7B shape at 128K, fold 8.  The widest activation operand is the W2
    # product's [B*T][G*Fs] (G = 4 shards of 1376 FFN columns): B*T*5504*2
    # bytes stay within 2^31 up to B = 11.
    (synth.get_config("7b_s128k").with_(batch=11), True, None),
    (synth.get_config("7b_s128k").with_(batch=12), False, "activation GEMM operand"),
    (synth.get_config("7b_s128k").with_(batch=33), False, "activation GEMM operand"),
    # fp32 at 64K: 4-byte elements, B*T*5504*4 bytes, up to B = 11
    (C3.with_(dtype="f32", batch=11), True, None),
    (C3.with_(dtype="f32", batch=12), False, "activation GEMM operand"),
])
def test_shapes_past_32bit_offsets_are_refused(cfg, ok, what):
    """The kernels address each buffer with 32-bit byte offsets and mark
    out-of-matrix rows with offset 2^31, so every buffer they stage from must
    span at most 2^31 bytes.  Larger shapes return TSP_E_SHAPE from the dims
    alone (no workspace size, nothing enqueued).  With H % D == 0 the K and
    V^T planes (B*S*d elements at most) never outgrow the activations
    (B*T*h = B*S*d*H/D), so the activation operand is the first limit."""
    d = tsp.make_dims(cfg, cfg.ranks[0])
    ws = tsp.workspace_bytes(d, tsp.TSP_WS_LAYER)
    if ok:
        assert ws > 0, tsp.lib().tsp_last_error()
        return
    assert ws == 0
    rc = _call_attn(d)
    assert tsp.STATUS[rc] == "TSP_E_SHAPE", rc
    assert what in tsp.lib().tsp_last_error().decode()
    L = tsp.lib()
    arr = (ctypes.c_void_p * cfg.fold)(*([4096] * cfg.fold))
    for call in (lambda: L.tsp_layer_shard(ctypes.byref(d), 16, 16, arr, 16, 16, arr, 16, 16, 1 << 40,
                                           None, None),
                 lambda: L.tsp_mlp_shard(ctypes.byref(d), 16, 16, arr, 16, 16, 1 << 40, None, None),
                 lambda: L.tsp_kv_shard(ctypes.byref(d), 16, 16, arr, 16, 16, 1 << 40, None)):
        assert tsp.STATUS[call()] == "TSP_E_SHAPE"


def test_noalloc_entry_point_refusals_on_the_host():
    """tsp_layer_shard_noalloc refuses, before any HIP call, dims whose layer
    workspace exceeds its static scratch (TSP_E_WORKSPACE) and the profiling
    flag (TSP_E_INVAL); bad dims give the usual codes."""
    L = tsp.lib()
    arr = (ctypes.c_void_p * 8)(*([4096] * 8))

    def call(d):
        return L.tsp_layer_shard_noalloc(ctypes.byref(d), 16, 16, arr, 16, 16, arr, 16, None, None)

    big = tsp.make_dims(C3, 3)
    assert tsp.workspace_bytes(big, tsp.TSP_WS_LAYER) > tsp.NOALLOC_SCRATCH_BYTES
    assert tsp.STATUS[call(big)] == "TSP_E_WORKSPACE"
    assert "static scratch" in L.tsp_last_error().decode()
    fits = tsp.make_dims(C3.with_(seq=4096), 3, tsp.TSP_F_SHARD_LAUNCH)
    assert tsp.workspace_bytes(fits, tsp.TSP_WS_LAYER) <= tsp.NOALLOC_SCRATCH_BYTES
    fits.flags |= tsp.TSP_F_PROFILE
    assert tsp.STATUS[call(fits)] == "TSP_E_INVAL"
    bad = tsp.make_dims(C3, 3)
    bad.rank = 9
    assert tsp.STATUS[call(bad)] == "TSP_E_INVAL"
    assert tsp.NOALLOC_SCRATCH_BYTES == 256 << 20


def test_clock_probe_argument_checks_on_the_host():
    L = tsp.lib()
    khz = ctypes.c_int32(0)
    assert tsp.STATUS[L.tsp_clock_probe(None, 8, 100, ctypes.byref(khz), None)] == "TSP_E_INVAL"
    assert tsp.STATUS[L.tsp_clock_probe(4096, 0, 100, ctypes.byref(khz), None)] == "TSP_E_INVAL"
    assert tsp.STATUS[L.tsp_clock_probe(4096, 100000, 100, ctypes.byref(khz), None)] == "TSP_E_INVAL"
    assert tsp.STATUS[L.tsp_clock_probe(4100, 8, 100, ctypes.byref(khz), None)] == "TSP_E_ALIGN"


def test_clock_from_probe_samples():
    """Shader cycles per wall tick times the wall rate: 100 MHz ticks and
    2.0e9 cycles per second read as 2000 MHz."""
    t = np.arange(0, 10) * 20000                  # 200 us apart at 100 MHz
    c = 5_000_000 + np.arange(0, 10) * 400_000    # 2 GHz
    mhz = tsp.clock_mhz(np.stack([t, c], axis=1).reshape(-1), 100_000)
    assert np.allclose(mhz, 2000.0)
