"""Python binding of libtp.so: one GPU's shard of a tensor-parallel transformer layer.

Argument marshalling only: every function takes torch CUDA tensors where the C
ABI takes device pointers, checks that each tensor is a contiguous CUDA tensor
large enough for what the library will touch, and calls the C function of the
same name on the current HIP stream. All computation runs in the library's HIP
kernels; there is no fallback. If libtp.so is missing the import succeeds but
every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "TP_DTYPE_F32", "TP_DTYPE_BF16", "TPError", "lib", "lib_path", "tp_linear_col",
    "tp_linear_row_partial", "tp_mlp_shard", "tp_mlp_shard_noalloc", "tp_ffn_gelu_shard", "tp_attn_proj_shard", "tp_combine_concat",
    "tp_combine_sum", "tp_shard_weight", "tp_shard_qkv", "tp_shard_weight_block", "tp_combine_concat_v",
    "kv_heads_per_shard", "tp_attn_core_shard", "tp_attn_decode_shard", "tp_release_workspaces",
    "tp_workspace_reserve", "tp_workspace_reserved", "tp_plan", "tp_status_string", "TP_ERR_WORKSPACE",
    "EXPORTS",
]

TP_DTYPE_F32 = 0
TP_DTYPE_BF16 = 1
TP_ERR_WORKSPACE = 7
_DT = {torch.float32: TP_DTYPE_F32, torch.bfloat16: TP_DTYPE_BF16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_SIGS = {
    "tp_linear_col": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp],
    "tp_linear_row_partial": [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp],
    "tp_mlp_shard": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp],
    "tp_mlp_shard_noalloc": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp],
    "tp_ffn_gelu_shard": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp],
    "tp_attn_proj_shard": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i32, _i32,
                           _i32, _vp],
    "tp_combine_concat": [ctypes.POINTER(_vp), _i32, ctypes.POINTER(_i64), _i32, _vp, _i64, _i32, _vp],
    "tp_combine_sum": [ctypes.POINTER(_vp), _i32, _i32, _vp, _vp, _i64, _i64, _i32, _vp],
    "tp_shard_weight": [_vp, _i64, _i64, _i32, _i32, _i32, _vp, _i32, _vp],
    "tp_shard_qkv": [_vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _vp],
    "tp_shard_weight_block": [_vp, _i64, _i64, _i32, _i64, _i64, _vp, _i32, _vp],
    "tp_attn_core_shard": [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _vp],
    "tp_attn_decode_shard": [_vp, _vp, _vp, _i64, _i64, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp],
    "tp_combine_concat_v": [ctypes.POINTER(_vp), _i32, ctypes.POINTER(_i64), _vp, _i64, _i32, _vp],
    "tp_workspace_reserve": [_vp, _sz, _sz],
    "tp_workspace_reserved": [_vp, ctypes.POINTER(_sz), ctypes.POINTER(_sz)],
    "tp_plan_begin": [],
    "tp_plan_end": [ctypes.POINTER(_sz), ctypes.POINTER(_sz)],
    "tp_release_workspaces": [],
    "tp_status_string": [_i32],
}
EXPORTS = tuple(_SIGS)


class TPError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {tp_status_string(status)}")


def lib_path() -> str:
    return os.path.join(_HERE, "libtp.so")


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m tensor_transformer_linear_col_amd.build`")
        handle = ctypes.CDLL(path)
        for name, args in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "tp_status_string" else ctypes.c_int32
        _LIB = handle
    return _LIB


def tp_status_string(status: int) -> str:
    return lib().tp_status_string(int(status)).decode()


def _call(name: str, *args) -> None:
    status = getattr(lib(), name)(*args)
    if status != 0:
        raise TPError(status, name)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _same(dt: int, **tensors) -> int:
    """Every given tensor (None skipped) must have the dtype `dt` the call passes to the
    library: a tensor of another width would be read or written out of bounds."""
    for name, t in tensors.items():
        if t is not None and _dt(t) != dt:
            raise TypeError(f"{name} is {t.dtype}, the call computes in "
                            f"{'float32' if dt == TP_DTYPE_F32 else 'bfloat16'}")
    return dt


def _pdt(P_r, partial_dtype, default: int) -> int:
    """Partial dtype: the explicit one (which P_r must then have), else P_r's, else default."""
    if partial_dtype is None:
        return _dt(P_r) if P_r is not None else default
    if P_r is not None and _dt(P_r) != partial_dtype:
        raise TypeError(f"P_r is {P_r.dtype} but partial_dtype is {partial_dtype}")
    return int(partial_dtype)


def _dev(t: torch.Tensor | None, name: str, min_numel: int | None = None) -> int:
    """Device pointer of a contiguous CUDA tensor holding at least min_numel elements."""
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {min_numel}")
    return t.data_ptr()


def _div(a: int, p: int):
    return a // p if p > 0 and a % p == 0 else None


def kv_heads_per_shard(n_kv_heads: int, tp_size: int):
    """KV heads one shard holds: G/p when p divides G, one (replicated) when p is a multiple
    of G, None otherwise (the library then returns TP_ERR_INDIVISIBLE)."""
    if tp_size <= 0 or n_kv_heads <= 0:
        return None
    if n_kv_heads % tp_size == 0:
        return n_kv_heads // tp_size
    return 1 if tp_size % n_kv_heads == 0 else None


def tp_linear_col(X, W_r, b_r, Y_r, M: int, in_features: int, out_features: int, tp_size: int) -> None:
    """Y_r = X W_r^T + b_r (shard of a column-parallel linear)."""
    dt = _same(_dt(X), W_r=W_r, b_r=b_r, Y_r=Y_r)
    n = _div(out_features, tp_size)
    need = n is not None and M > 0
    _call("tp_linear_col",
          _dev(X, "X", M * in_features if need else None),
          _dev(W_r, "W_r", n * in_features if need else None),
          _dev(b_r, "b_r", n if need else None),
          _dev(Y_r, "Y_r", M * n if need else None),
          M, in_features, out_features, tp_size, dt, _stream())


def tp_linear_row_partial(X_r, ldx: int, W_r, P_r, M: int, in_features: int, out_features: int,
                          tp_size: int, partial_dtype=None) -> None:
    """P_r = X_r W_r^T (partial of a row-parallel linear, no bias).

    X_r may be a view into a larger CUDA tensor (row stride ldx); it is passed as
    its data pointer and must reach (M-1)*ldx + in_features/p elements.
    """
    dt = _same(_dt(W_r), X_r=X_r)
    k = _div(in_features, tp_size)
    pdt = _pdt(P_r, partial_dtype, dt)
    need = k is not None and M > 0 and ldx >= (k or 0)
    if not isinstance(X_r, torch.Tensor) or not X_r.is_cuda:
        raise ValueError("X_r must be a CUDA tensor")
    if need:
        storage_left = X_r.untyped_storage().nbytes() // X_r.element_size() - X_r.storage_offset()
        if storage_left < (M - 1) * ldx + k:
            raise ValueError("X_r does not reach the last row")
    _call("tp_linear_row_partial", X_r.data_ptr(), ldx,
          _dev(W_r, "W_r", out_features * k if need else None),
          _dev(P_r, "P_r", M * out_features if need else None),
          M, in_features, out_features, tp_size, dt, pdt, _stream())


def tp_mlp_shard(X, Wg_r, Wu_r, bg_r, bu_r, Wd_r, H_r, P_r, M: int, hidden: int, intermediate: int,
                 tp_size: int, partial_dtype=None, _name: str = "tp_mlp_shard") -> None:
    """H_r = silu(X Wg_r^T + bg_r) * (X Wu_r^T + bu_r); P_r = H_r Wd_r^T (partial)."""
    i = _div(intermediate, tp_size)
    need = i is not None and M > 0
    dt = _same(_dt(X), Wg_r=Wg_r, Wu_r=Wu_r, bg_r=bg_r, bu_r=bu_r, Wd_r=Wd_r, H_r=H_r)
    pdt = _pdt(P_r, partial_dtype, dt)
    _call(_name,
          _dev(X, "X", M * hidden if need else None),
          _dev(Wg_r, "Wg_r", i * hidden if need else None),
          _dev(Wu_r, "Wu_r", i * hidden if need else None),
          _dev(bg_r, "bg_r", i if need else None),
          _dev(bu_r, "bu_r", i if need else None),
          _dev(Wd_r, "Wd_r", hidden * i if need and P_r is not None else None),
          _dev(H_r, "H_r", M * i if need else None),
          _dev(P_r, "P_r", M * hidden if need else None),
          M, hidden, intermediate, tp_size, dt, pdt, _stream())


def tp_mlp_shard_noalloc(X, Wg_r, Wu_r, bg_r, bu_r, Wd_r, H_r, P_r, M: int, hidden: int, intermediate: int,
                         tp_size: int, partial_dtype=None) -> None:
    """tp_mlp_shard without a reserved work space: its split reductions use the library's fixed
    per-GPU scratch array (calls that overlap on one GPU race)."""
    tp_mlp_shard(X, Wg_r, Wu_r, bg_r, bu_r, Wd_r, H_r, P_r, M, hidden, intermediate, tp_size, partial_dtype,
                 _name="tp_mlp_shard_noalloc")


def tp_ffn_gelu_shard(X, W1_r, b1_r, W2_r, H_r, P_r, M: int, hidden: int, intermediate: int,
                      tp_size: int, partial_dtype=None) -> None:
    """H_r = gelu(X W1_r^T + b1_r) (erf form); P_r = H_r W2_r^T (partial)."""
    i = _div(intermediate, tp_size)
    need = i is not None and M > 0
    dt = _same(_dt(X), W1_r=W1_r, b1_r=b1_r, W2_r=W2_r, H_r=H_r)
    pdt = _pdt(P_r, partial_dtype, dt)
    _call("tp_ffn_gelu_shard",
          _dev(X, "X", M * hidden if need else None),
          _dev(W1_r, "W1_r", i * hidden if need else None),
          _dev(b1_r, "b1_r", i if need else None),
          _dev(W2_r, "W2_r", hidden * i if need and P_r is not None else None),
          _dev(H_r, "H_r", M * i if need else None),
          _dev(P_r, "P_r", M * hidden if need else None),
          M, hidden, intermediate, tp_size, dt, pdt, _stream())


def tp_attn_proj_shard(X, Wqkv_r, bqkv_r, QKV_r, A_r, Wo_r, P_r, M: int, hidden: int, n_heads: int,
                       n_kv_heads: int, head_dim: int, tp_size: int, partial_dtype=None) -> None:
    """QKV_r = X Wqkv_r^T + bqkv_r; P_r = A_r Wo_r^T (partial). Either half may be skipped (None)."""
    hq, hk = _div(n_heads, tp_size), kv_heads_per_shard(n_kv_heads, tp_size)
    need = hq is not None and hk is not None and M > 0
    nqkv = (hq + 2 * hk) * head_dim if need else 0
    ka = hq * head_dim if need else 0
    ref = X if X is not None else A_r
    dt = _same(_dt(ref), X=X, Wqkv_r=Wqkv_r, bqkv_r=bqkv_r, QKV_r=QKV_r, A_r=A_r, Wo_r=Wo_r)
    pdt = _pdt(P_r, partial_dtype, dt)
    q_need = need and QKV_r is not None
    o_need = need and P_r is not None
    _call("tp_attn_proj_shard",
          _dev(X, "X", M * hidden if q_need else None),
          _dev(Wqkv_r, "Wqkv_r", nqkv * hidden if q_need else None),
          _dev(bqkv_r, "bqkv_r", nqkv if q_need else None),
          _dev(QKV_r, "QKV_r", M * nqkv if q_need else None),
          _dev(A_r, "A_r", M * ka if o_need else None),
          _dev(Wo_r, "Wo_r", hidden * ka if o_need else None),
          _dev(P_r, "P_r", M * hidden if o_need else None),
          M, hidden, n_heads, n_kv_heads, head_dim, tp_size, dt, pdt, _stream())


def tp_combine_concat(shards, seg_widths, Y, M: int) -> None:
    """Y = per-segment concat of the shards in rank order."""
    p = len(shards)
    s = int(sum(seg_widths))
    dt = _same(_dt(Y), **{f"shards[{r}]": t for r, t in enumerate(shards)})
    ptrs = (ctypes.c_void_p * p)(*[_dev(t, f"shards[{r}]", M * s) for r, t in enumerate(shards)])
    segs = (ctypes.c_int64 * len(seg_widths))(*[int(w) for w in seg_widths])
    _call("tp_combine_concat", ptrs, p, segs, len(seg_widths), _dev(Y, "Y", M * p * s), M, dt,
          _stream())


def tp_combine_sum(partials, b, Y, M: int, N: int) -> None:
    """Y = sum_r partials[r] + b (bias once), fp32 accumulation in rank order."""
    p = len(partials)
    pdt = _same(_dt(partials[0]), **{f"partials[{r}]": t for r, t in enumerate(partials)})
    odt = _same(_dt(Y), b=b)
    ptrs = (ctypes.c_void_p * p)(*[_dev(t, f"partials[{r}]", M * N) for r, t in enumerate(partials)])
    _call("tp_combine_sum", ptrs, p, pdt, _dev(b, "b", N), _dev(Y, "Y", M * N), M, N, odt, _stream())


def tp_shard_weight(W, out_features: int, in_features: int, tp_size: int, rank: int, axis: int,
                    W_r) -> None:
    """W_r = the rank's block of W along axis 0 (output rows) or 1 (input columns)."""
    dt = _same(_dt(W), W_r=W_r)
    _call("tp_shard_weight", _dev(W, "W", out_features * in_features), out_features, in_features,
          tp_size, rank, axis, _dev(W_r, "W_r", (out_features * in_features) // max(tp_size, 1)),
          dt, _stream())


def tp_shard_qkv(Wqkv, in_features: int, n_heads: int, n_kv_heads: int, head_dim: int, tp_size: int,
                 rank: int, Wqkv_r) -> None:
    """Wqkv_r = rows of the rank's Q heads, then K heads, then V heads (a KV head is
    replicated on tp_size / n_kv_heads shards when there are more shards than KV heads)."""
    dt = _same(_dt(Wqkv), Wqkv_r=Wqkv_r)
    rows = (n_heads + 2 * n_kv_heads) * head_dim
    hq, hk = _div(n_heads, tp_size), kv_heads_per_shard(n_kv_heads, tp_size)
    shard_rows = (hq + 2 * hk) * head_dim if hq is not None and hk is not None else None
    _call("tp_shard_qkv", _dev(Wqkv, "Wqkv", rows * in_features), in_features, n_heads, n_kv_heads,
          head_dim, tp_size, rank, _dev(Wqkv_r, "Wqkv_r", shard_rows * in_features if shard_rows else None),
          dt, _stream())


def tp_attn_core_shard(QKV_r, A_r, M: int, n_heads: int, n_kv_heads: int, head_dim: int, tp_size: int,
                       causal: bool = True) -> None:
    """A_r = head-local (grouped-query, optionally causal) attention over QKV_r's Q | K | V."""
    dt = _same(_dt(QKV_r), A_r=A_r)
    hq, hk = _div(n_heads, tp_size), kv_heads_per_shard(n_kv_heads, tp_size)
    need = hq is not None and hk is not None and M > 0
    nqkv = (hq + 2 * hk) * head_dim if need else 0
    _call("tp_attn_core_shard", _dev(QKV_r, "QKV_r", M * nqkv if need else None),
          _dev(A_r, "A_r", M * hq * head_dim if need else None), M, n_heads, n_kv_heads, head_dim, tp_size,
          1 if causal else 0, dt, _stream())


def tp_attn_decode_shard(QKV_r, K_cache_r, V_cache_r, cache_len: int, A_r, M: int, n_heads: int,
                         n_kv_heads: int, head_dim: int, tp_size: int) -> None:
    """Append the M new tokens' K/V rows of QKV_r to the shard's caches at cache_len, then
    A_r = causal attention of the new tokens over the cache and themselves. The caches are
    [capacity, hk*head_dim] tensors; the capacity is read from K_cache_r's size."""
    dt = _same(_dt(QKV_r), K_cache_r=K_cache_r, V_cache_r=V_cache_r, A_r=A_r)
    hq, hk = _div(n_heads, tp_size), kv_heads_per_shard(n_kv_heads, tp_size)
    need = hq is not None and hk is not None
    nqkv = (hq + 2 * hk) * head_dim if need else 0
    ldkv = hk * head_dim if need else 0
    capacity = K_cache_r.numel() // ldkv if need and ldkv > 0 else 0
    _call("tp_attn_decode_shard", _dev(QKV_r, "QKV_r", M * nqkv if need else None),
          _dev(K_cache_r, "K_cache_r", capacity * ldkv if need else None),
          _dev(V_cache_r, "V_cache_r", capacity * ldkv if need else None), cache_len, capacity,
          _dev(A_r, "A_r", M * hq * head_dim if need else None), M, n_heads, n_kv_heads, head_dim, tp_size,
          dt, _stream())


def tp_shard_weight_block(W, out_features: int, in_features: int, axis: int, start: int, width: int,
                          W_r) -> None:
    """W_r = W[start:start+width, :] (axis 0) or W[:, start:start+width] (axis 1), any width."""
    dt = _same(_dt(W), W_r=W_r)
    n_r = (width * in_features if axis == 0 else out_features * width) if width > 0 else None
    _call("tp_shard_weight_block", _dev(W, "W", out_features * in_features), out_features, in_features,
          axis, start, width, _dev(W_r, "W_r", n_r), dt, _stream())


def tp_combine_concat_v(shards, widths, Y, M: int) -> None:
    """Y = [shards[0] | shards[1] | ...] with per-shard widths (an uneven column split)."""
    n = len(shards)
    total = int(sum(widths))
    dt = _same(_dt(Y), **{f"shards[{r}]": t for r, t in enumerate(shards)})
    ptrs = (ctypes.c_void_p * n)(*[_dev(t, f"shards[{r}]", M * int(widths[r])) for r, t in enumerate(shards)])
    ws = (ctypes.c_int64 * n)(*[int(w) for w in widths])
    _call("tp_combine_concat_v", ptrs, n, ws, _dev(Y, "Y", M * total), M, dt, _stream())


def tp_workspace_reserve(partial_bytes: int, n_counters: int) -> None:
    """Reserve the work space of the current device and stream (setup only: it may allocate
    and synchronise the stream; never call it while the stream is being captured)."""
    _call("tp_workspace_reserve", _stream(), int(partial_bytes), int(n_counters))


def tp_workspace_reserved() -> tuple[int, int]:
    """(partial bytes, counters) reserved for the current device and stream."""
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _call("tp_workspace_reserved", _stream(), ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


class tp_plan:
    """Dry run: inside `with tp_plan() as need:` every call validates and plans its launches
    but enqueues nothing; on exit need.partial_bytes / need.n_counters hold the largest work
    space any of them needs (pass them to tp_workspace_reserve)."""

    def __enter__(self):
        self.partial_bytes = 0
        self.n_counters = 0
        _call("tp_plan_begin")
        return self

    def __exit__(self, *exc):
        a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
        _call("tp_plan_end", ctypes.byref(a), ctypes.byref(b))
        self.partial_bytes, self.n_counters = a.value, b.value
        return False


def tp_release_workspaces() -> None:
    _call("tp_release_workspaces")
