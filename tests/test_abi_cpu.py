"""The C ABI on the CPU: the library loads, exports every declared function, and
rejects bad arguments on the host before any HIP call (fake, never-dereferenced
pointers are enough for that). No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import tensor_transformer_linear_col_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_linear.h")

OK, NULL, SHAPE, INDIV, DTYPE, ALIGN, HIP, WORKSPACE = range(8)
F32, BF16 = 0, 1
P = 0x100000  # a 16-byte aligned fake device address, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:tp_status_t|const char\*)\s+(tp_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tp.lib_path()):
        pytest.skip("libtp.so not built")
    return tp.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) == 20, names
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(tp.EXPORTS)


def test_status_strings(L):
    for code in range(8):
        assert tp.tp_status_string(code).startswith(
            ["TP_OK", "TP_ERR_NULL", "TP_ERR_SHAPE", "TP_ERR_INDIVISIBLE", "TP_ERR_DTYPE",
             "TP_ERR_ALIGN", "TP_ERR_HIP", "TP_ERR_WORKSPACE"][code])
    assert "unknown" in tp.tp_status_string(99)


def col(L, X=P, W=P, b=0, Y=P, M=4, K=4096, N=11008, p=2, dt=BF16):
    return L.tp_linear_col(X, W, b, Y, M, K, N, p, dt, None)


def test_linear_col_errors(L):
    assert col(L, X=0) == NULL
    assert col(L, W=0) == NULL
    assert col(L, Y=0) == NULL
    assert col(L, N=11008, p=3) == INDIV           # the listing's out_features % world_size assert
    assert col(L, p=0) == SHAPE
    assert col(L, p=65) == SHAPE
    assert col(L, M=-1) == SHAPE
    assert col(L, K=0) == SHAPE
    assert col(L, N=0) == SHAPE
    assert col(L, dt=7) == DTYPE
    assert col(L, X=P + 8) == ALIGN                # bf16 operand read with 16-byte loads
    assert col(L, K=4100) == ALIGN                 # row stride 8200 B is not a multiple of 16
    assert col(L, M=0) == OK                       # nothing to do: returns before any HIP call
    # fp32 has no alignment rule (the toy's 3-wide shards)
    assert col(L, X=P + 4, K=8, N=6, p=2, dt=F32, M=0) == OK


def row(L, X=P, ldx=None, W=P, Y=P, M=4, K=11008, N=4096, p=2, dt=BF16, pdt=BF16):
    ldx = K // p if ldx is None else ldx
    return L.tp_linear_row_partial(X, ldx, W, Y, M, K, N, p, dt, pdt, None)


def test_linear_row_partial_errors(L):
    assert row(L, X=0) == NULL
    assert row(L, K=11008, p=3, ldx=4000) == INDIV   # in_features % world_size
    assert row(L, ldx=5503) == SHAPE                 # ldx < in_features / p
    assert row(L, dt=F32, pdt=BF16) == DTYPE         # fp32 inputs need fp32 partials
    assert row(L, pdt=3) == DTYPE
    assert row(L, ldx=5505) == ALIGN
    assert row(L, M=0) == OK
    assert row(L, M=0, pdt=F32) == OK                # bf16 inputs may keep fp32 partials


def mlp(L, X=P, Wg=P, Wu=P, bg=0, bu=0, Wd=P, H=P, Pr=P, M=1, h=4096, i=11008, p=2, dt=BF16, pdt=BF16):
    return L.tp_mlp_shard(X, Wg, Wu, bg, bu, Wd, H, Pr, M, h, i, p, dt, pdt, None)


def test_mlp_shard_errors(L):
    assert mlp(L, H=0) == NULL
    assert mlp(L, Wd=0) == NULL
    assert mlp(L, bg=P) == NULL                      # gate and up biases come together
    assert mlp(L, i=11008, p=3) == INDIV
    assert mlp(L, i=28672, p=5) == INDIV
    assert mlp(L, Wg=P + 2) == ALIGN
    assert mlp(L, dt=F32, pdt=BF16) == DTYPE
    assert mlp(L, M=0) == OK
    assert mlp(L, M=0, Wd=0, Pr=0) == OK             # down projection skipped


def gelu_ffn(L, X=P, W1=P, b1=0, W2=P, H=P, Pr=P, M=4, h=4096, i=11008, p=2, dt=BF16, pdt=BF16):
    return L.tp_ffn_gelu_shard(X, W1, b1, W2, H, Pr, M, h, i, p, dt, pdt, None)


def test_ffn_gelu_shard_errors(L):
    assert gelu_ffn(L, X=0) == NULL
    assert gelu_ffn(L, W1=0) == NULL
    assert gelu_ffn(L, H=0) == NULL
    assert gelu_ffn(L, W2=0) == NULL                 # the row layer needs its weights
    assert gelu_ffn(L, i=11008, p=3) == INDIV        # the listing's divisibility assert
    assert gelu_ffn(L, p=0) == SHAPE
    assert gelu_ffn(L, W1=P + 2) == ALIGN
    assert gelu_ffn(L, dt=F32, pdt=BF16) == DTYPE
    assert gelu_ffn(L, M=0) == OK
    assert gelu_ffn(L, M=0, W2=0, Pr=0) == OK        # row layer skipped


def attn(L, X=P, Wqkv=P, b=0, QKV=P, A=P, Wo=P, Pr=P, M=1, h=8192, nh=64, nkv=8, d=128, p=8,
         dt=BF16, pdt=BF16):
    return L.tp_attn_proj_shard(X, Wqkv, b, QKV, A, Wo, Pr, M, h, nh, nkv, d, p, dt, pdt, None)


def test_uneven_split_entry_points_errors(L):
    blk = lambda **k: L.tp_shard_weight_block(k.get("W", P), k.get("out", 9), k.get("inn", 8), k.get("axis", 0),
                                              k.get("start", 5), k.get("width", 4), k.get("Wr", P), k.get("dt", F32), None)
    assert blk(W=0) == NULL
    assert blk(start=6) == SHAPE                     # block leaves the 9 output rows
    assert blk(width=0) == SHAPE
    assert blk(axis=2) == SHAPE
    assert blk(axis=1, start=8, width=1) == SHAPE
    ptrs = (ctypes.c_void_p * 2)(P, P)
    ws = (ctypes.c_int64 * 2)(5, 4)
    assert L.tp_combine_concat_v(ptrs, 2, ws, P, 0, F32, None) == OK
    assert L.tp_combine_concat_v(ptrs, 0, ws, P, 1, F32, None) == SHAPE
    bad = (ctypes.c_int64 * 2)(5, 0)
    assert L.tp_combine_concat_v(ptrs, 2, bad, P, 1, F32, None) == SHAPE
    assert L.tp_combine_concat_v(ptrs, 2, ws, 0, 1, F32, None) == NULL


def test_attn_core_shard_errors(L):
    core = lambda **k: L.tp_attn_core_shard(k.get("Q", P), k.get("A", P), k.get("M", 16), k.get("nh", 64),
                                            k.get("nkv", 8), k.get("d", 128), k.get("p", 8), 1, k.get("dt", BF16), None)
    assert core(Q=0) == NULL
    assert core(dt=F32) == DTYPE                     # bf16 only
    assert core(d=96) == SHAPE
    assert core(p=3) == INDIV
    assert core(nh=48, nkv=8, p=12) == INDIV
    assert core(nh=24, nkv=16, p=8) == INDIV         # 3 query heads cannot group over 2 KV heads
    assert core(Q=P + 8) == ALIGN
    assert core(M=0) == OK
    assert core(M=0, nkv=8, p=16) == OK              # KV heads replicated


def test_attn_decode_shard_errors(L):
    dec = lambda **k: L.tp_attn_decode_shard(k.get("Q", P), k.get("Kc", P), k.get("Vc", P), k.get("T", 100),
                                             k.get("cap", 4096), k.get("A", P), k.get("M", 1), k.get("nh", 64),
                                             k.get("nkv", 8), k.get("d", 128), k.get("p", 8), k.get("dt", BF16), None)
    assert dec(Kc=0) == NULL
    assert dec(Vc=0) == NULL
    assert dec(dt=F32) == DTYPE
    assert dec(d=80) == SHAPE
    assert dec(T=-1) == SHAPE
    assert dec(T=4096, M=1) == SHAPE                 # no room left in the cache
    assert dec(T=4000, M=97) == SHAPE
    assert dec(p=3) == INDIV
    assert dec(Kc=P + 8) == ALIGN
    assert dec(nkv=64, p=64, nh=64, T=1 << 23, cap=(1 << 23) + 8, M=1) == SHAPE  # 2 GiB of cache
    assert dec(M=0) == OK                            # nothing to append or attend
    assert dec(M=0, T=4096) == OK


def test_attn_proj_shard_errors(L):
    assert attn(L, p=3) == INDIV                     # TP size must divide the heads
    assert attn(L, nh=48, nkv=8, p=12) == INDIV      # ... and divide, or be a multiple of, the KV heads
    assert attn(L, nkv=8, p=16, M=0) == OK           # 16 shards, 8 KV heads: each replicated twice
    assert attn(L, A=0) == NULL
    assert attn(L, QKV=0, X=0, Wqkv=0, M=0) == OK    # QKV half skipped
    assert attn(L, Pr=0, A=0, Wo=0, M=0) == OK       # O half skipped
    assert attn(L, d=0) == SHAPE
    assert attn(L, M=0) == OK


def test_combine_errors(L):
    ptrs = (ctypes.c_void_p * 2)(P, P)
    bad = (ctypes.c_void_p * 2)(P, 0)
    segs = (ctypes.c_int64 * 3)(1024, 128, 128)
    assert L.tp_combine_concat(None, 2, segs, 3, P, 4, BF16, None) == NULL
    assert L.tp_combine_concat(bad, 2, segs, 3, P, 4, BF16, None) == NULL
    assert L.tp_combine_concat(ptrs, 2, segs, 0, P, 4, BF16, None) == SHAPE
    assert L.tp_combine_concat(ptrs, 2, segs, 9, P, 4, BF16, None) == SHAPE
    assert L.tp_combine_concat(ptrs, 0, segs, 3, P, 4, BF16, None) == SHAPE
    assert L.tp_combine_concat(ptrs, 2, segs, 3, P, 4, 5, None) == DTYPE
    zero = (ctypes.c_int64 * 1)(0)
    assert L.tp_combine_concat(ptrs, 2, zero, 1, P, 4, BF16, None) == SHAPE
    assert L.tp_combine_sum(None, 2, BF16, 0, P, 4, 4096, BF16, None) == NULL
    assert L.tp_combine_sum(bad, 2, BF16, 0, P, 4, 4096, BF16, None) == NULL
    assert L.tp_combine_sum(ptrs, 2, BF16, 0, 0, 4, 4096, BF16, None) == NULL
    assert L.tp_combine_sum(ptrs, 2, BF16, 0, P, 4, 0, BF16, None) == SHAPE
    assert L.tp_combine_sum(ptrs, 2, 9, 0, P, 4, 4096, BF16, None) == DTYPE
    assert L.tp_combine_sum(ptrs, 99, BF16, 0, P, 4, 4096, BF16, None) == SHAPE


def test_shard_errors(L):
    assert L.tp_shard_weight(0, 6, 8, 2, 0, 0, P, F32, None) == NULL
    assert L.tp_shard_weight(P, 6, 8, 2, 2, 0, P, F32, None) == SHAPE   # rank >= p
    assert L.tp_shard_weight(P, 6, 8, 2, -1, 0, P, F32, None) == SHAPE
    assert L.tp_shard_weight(P, 6, 8, 2, 0, 2, P, F32, None) == SHAPE   # axis
    assert L.tp_shard_weight(P, 9, 8, 2, 0, 0, P, F32, None) == INDIV   # 9 outputs over 2 shards
    assert L.tp_shard_weight(P, 6, 9, 2, 0, 1, P, F32, None) == INDIV
    assert L.tp_shard_qkv(P, 8192, 64, 8, 128, 3, 0, P, BF16, None) == INDIV
    assert L.tp_shard_qkv(P, 8192, 64, 8, 128, 8, 8, P, BF16, None) == SHAPE


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 8)
    with pytest.raises(ValueError):
        tp.tp_linear_col(x, x, None, x, 1, 8, 6, 2)


# ---- work space: sized by a dry run, reserved by the caller, never allocated by a call ----

def _plan(L, fn):
    """Dry run of fn(): its status and the work space (partial bytes, counters) it plans."""
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert L.tp_plan_begin() == OK
    try:
        st = fn()
    finally:
        assert L.tp_plan_end(ctypes.byref(a), ctypes.byref(b)) == OK
    return st, a.value, b.value


def test_dry_run_sizes_the_split_reductions(L):
    """A dry run validates, enqueues nothing (no GPU here, so any launch would fail with
    TP_ERR_HIP) and reports the largest work space of the calls inside it. Without a device
    the library plans for 256 compute units, as on MI355X."""
    # A 1320-feature column shard at 1000 tokens, K = 16384: its 9 x 8 = 72 tiles of 160 x 128 in
    # 3 K ranges would fill only 216 of 256 CUs, so 6 x 4 = 24 tiles of 256 x 256 run, each cut
    # into 8 K ranges -> 192 fp32 partial tiles of 256 KB.
    big = lambda: col(L, M=1000, K=16384, N=2640, p=2)
    assert _plan(L, big) == (OK, 192 * 256 * 256 * 4, 0)
    # 70B QKV shard at TP = 8 and 2048 tokens: 8 x 16 = 128 tiles of 160 x 128, each cut into 2 K
    # ranges -> 256 partial tiles of 80 KB; at 1024 tokens 64 tiles in 4 ranges, the same.
    qkv = lambda: L.tp_attn_proj_shard(P, P, 0, P, 0, 0, 0, 2048, 8192, 64, 8, 128, 8, BF16, BF16, None)
    assert _plan(L, qkv) == (OK, 256 * 160 * 128 * 4, 0)
    qkv1k = lambda: L.tp_attn_proj_shard(P, P, 0, P, 0, 0, 0, 1024, 8192, 64, 8, 128, 8, BF16, BF16, None)
    assert _plan(L, qkv1k) == (OK, 256 * 160 * 128 * 4, 0)
    # At 4096 tokens its 8 x 32 = 256 tiles of 160 x 128 fill the chip: no split, no work space.
    qkv4k = lambda: L.tp_attn_proj_shard(P, P, 0, P, 0, 0, 0, 4096, 8192, 64, 8, 128, 8, BF16, BF16, None)
    assert _plan(L, qkv4k) == (OK, 0, 0)
    # The same QKV shard at 8 tokens: 40 row groups of 32 outputs, K cut in 7 -> 280
    # workgroups with two 2 KB partial tiles each, and one arrival counter per row group.
    qkv1 = lambda: L.tp_attn_proj_shard(P, P, 0, P, 0, 0, 0, 8, 8192, 64, 8, 128, 8, BF16, BF16, None)
    assert _plan(L, qkv1) == (OK, 280 * 2 * 512 * 4, 40)
    # At 1 to 4 tokens the GEMV kernel splits the features across workgroups, not K.
    for m in (1, 4):
        assert _plan(L, lambda: L.tp_attn_proj_shard(P, P, 0, P, 0, 0, 0, m, 8192, 64, 8, 128, 8, BF16, BF16,
                                                     None)) == (OK, 0, 0)
    # Products that split nothing need no work space; M = 0 does nothing at all.
    gateup = lambda: L.tp_mlp_shard(P, P, P, 0, 0, P, P, P, 4096, 8192, 28672, 8, BF16, BF16, None)
    assert _plan(L, gateup) == (OK, 0, 0)
    assert _plan(L, lambda: col(L, M=0)) == (OK, 0, 0)
    # Several calls: the largest need of any of them.
    both = lambda: (qkv1(), big(), qkv(), gateup())[-1]
    assert _plan(L, both) == (OK, 192 * 256 * 256 * 4, 40)
    # Validation still applies inside a dry run.
    assert _plan(L, lambda: col(L, X=0))[0] == NULL


def test_multi_launch_call_rejects_before_its_first_launch(L):
    """tp_mlp_shard whose gate/up product is fine but whose down product would need 32-bit
    offsets past 4 GiB (M x I/p x 2 bytes) is rejected as a whole before anything is
    enqueued: it returns TP_ERR_SHAPE, not the TP_ERR_HIP a launch attempt gives here."""
    M, hidden, inter = 1 << 20, 1024, 2048
    st = L.tp_mlp_shard(P, P, P, 0, 0, P, P, P, M, hidden, inter, 1, BF16, BF16, None)
    assert st == SHAPE
    # Without the down product the same call plans fine (and then needs the GPU).
    assert _plan(L, lambda: L.tp_mlp_shard(P, P, P, 0, 0, 0, P, 0, M, hidden, inter, 1, BF16, BF16, None)) == (OK, 0, 0)


def test_workspace_calls_without_a_device(L):
    a, b = ctypes.c_size_t(7), ctypes.c_size_t(7)
    assert L.tp_workspace_reserved(None, ctypes.byref(a), ctypes.byref(b)) in (OK, HIP)
    assert L.tp_workspace_reserved(None, None, ctypes.byref(b)) == NULL
    # Inside a dry run a reservation does nothing (and needs no device).
    assert _plan(L, lambda: L.tp_workspace_reserve(None, 1 << 20, 64)) == (OK, 0, 0)


def test_binding_rejects_mismatched_dtypes_before_any_device_access():
    """Each wrapper passes one dtype per role to the library; a tensor of another width
    would be read or written out of bounds, so it raises TypeError first (CPU tensors
    suffice: the dtype check precedes the device checks)."""
    import torch
    f, b = torch.float32, torch.bfloat16
    t = lambda *shape, dt=b: torch.zeros(*shape, dtype=dt)
    with pytest.raises(TypeError, match="W_r"):
        tp.tp_linear_col(t(2, 8, dt=f), t(3, 8), None, t(2, 3, dt=f), 2, 8, 6, 2)
    with pytest.raises(TypeError, match="Y_r"):
        tp.tp_linear_col(t(2, 8), t(3, 8), None, t(2, 3, dt=f), 2, 8, 6, 2)
    with pytest.raises(TypeError, match="b_r"):
        tp.tp_linear_col(t(2, 8), t(3, 8), t(3, dt=f), t(2, 3), 2, 8, 6, 2)
    with pytest.raises(TypeError, match="X_r"):
        tp.tp_linear_row_partial(t(2, 4, dt=f), 4, t(6, 4), t(2, 6), 2, 8, 6, 2)
    with pytest.raises(TypeError, match="P_r"):
        tp.tp_linear_row_partial(t(2, 4), 4, t(6, 4), t(2, 6, dt=f), 2, 8, 6, 2, partial_dtype=tp.TP_DTYPE_BF16)
    with pytest.raises(TypeError, match="H_r"):
        tp.tp_mlp_shard(t(2, 8), t(4, 8), t(4, 8), None, None, None, t(2, 4, dt=f), None, 2, 8, 8, 2)
    with pytest.raises(TypeError, match="Wu_r"):
        tp.tp_mlp_shard(t(2, 8), t(4, 8), t(4, 8, dt=f), None, None, None, t(2, 4), None, 2, 8, 8, 2)
    with pytest.raises(TypeError, match="W2_r"):
        tp.tp_ffn_gelu_shard(t(2, 8), t(4, 8), None, t(8, 4, dt=f), t(2, 4), t(2, 8), 2, 8, 8, 2)
    with pytest.raises(TypeError, match="Wo_r"):
        tp.tp_attn_proj_shard(None, None, None, None, t(2, 16), t(8, 16, dt=f), t(2, 8), 2, 8, 2, 2, 8, 1)
    with pytest.raises(TypeError, match="partials"):
        tp.tp_combine_sum([t(2, 8), t(2, 8, dt=f)], None, t(2, 8), 2, 8)
    with pytest.raises(TypeError, match="b"):
        tp.tp_combine_sum([t(2, 8), t(2, 8)], t(8, dt=f), t(2, 8), 2, 8)
    with pytest.raises(TypeError, match="shards"):
        tp.tp_combine_concat([t(2, 8), t(2, 8, dt=f)], [8], t(2, 16), 2)
    with pytest.raises(TypeError, match="shards"):
        tp.tp_combine_concat_v([t(2, 8, dt=f), t(2, 8)], [8, 8], t(2, 16), 2)
    with pytest.raises(TypeError, match="W_r"):
        tp.tp_shard_weight(t(8, 8), 8, 8, 2, 0, 0, t(4, 8, dt=f))
    with pytest.raises(TypeError, match="Wqkv_r"):
        tp.tp_shard_qkv(t(48, 8), 8, 4, 2, 8, 2, 0, t(32, 8, dt=f))
    with pytest.raises(TypeError, match="W_r"):
        tp.tp_shard_weight_block(t(8, 8), 8, 8, 0, 0, 4, t(4, 8, dt=f))
    with pytest.raises(TypeError, match="A_r"):
        tp.tp_attn_core_shard(t(4, 256), t(4, 128, dt=f), 4, 2, 1, 64, 1)
    with pytest.raises(TypeError, match="V_cache_r"):
        tp.tp_attn_decode_shard(t(1, 256), t(8, 64), t(8, 64, dt=f), 0, t(1, 128), 1, 2, 1, 64, 1)
