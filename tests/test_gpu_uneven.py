"""GPU parity of uneven splits (explicit per-shard widths) and of KV-head replication when
there are more shards than KV heads, against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
import tensor_transformer_linear_col_amd as tp
import tp_inputs as I
from gpu_util import BF16_TOL, F32_TOL, dev, err, host64, log_case

pytestmark = pytest.mark.gpu


def test_shard_weight_block_is_exact():
    w = I.weight(1000, 64, seed=501)
    W = dev(w)
    for axis, (start, width) in [(0, (304, 256)), (0, (0, 8)), (1, (16, 40)), (1, (56, 8))]:
        shape = (width, 64) if axis == 0 else (1000, width)
        W_r = torch.empty(*shape, dtype=torch.bfloat16, device="cuda")
        tp.tp_shard_weight_block(W, 1000, 64, axis, start, width, W_r)
        torch.cuda.synchronize()
        ref = host64(w)[start:start + width, :] if axis == 0 else host64(w)[:, start:start + width]
        np.testing.assert_array_equal(host64(W_r), ref)


@pytest.mark.parametrize("M", [1, 40, 300])
def test_uneven_column_split_concat(M):
    K, widths = 1024, (304, 256, 440)
    N = sum(widths)
    log_case("uneven column split", M, K, widths)
    x, w, b = I.activations(M, K, 510 + M), I.weight(N, K, 511), I.bias(N, 512)
    X, W, B = dev(x), dev(w), dev(b)
    outs, start = [], 0
    for width in widths:
        W_r = torch.empty(width, K, dtype=torch.bfloat16, device="cuda")
        b_r = torch.empty(width, dtype=torch.bfloat16, device="cuda")
        tp.tp_shard_weight_block(W, N, K, 0, start, width, W_r)
        tp.tp_shard_weight_block(B, N, 1, 0, start, width, b_r)
        Y_r = torch.empty(M, width, dtype=torch.bfloat16, device="cuda")
        tp.tp_linear_col(X, W_r, b_r, Y_r, M, K, width, 1)
        outs.append(Y_r)
        start += width
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tp.tp_combine_concat_v(outs, widths, Y, M)
    torch.cuda.synchronize()
    assert err(Y, O.linear(host64(x), host64(w), host64(b))) <= BF16_TOL
    # the concat is a pure copy of the shards
    np.testing.assert_array_equal(host64(Y), np.concatenate([host64(o) for o in outs], axis=1))


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, BF16_TOL), (torch.float32, F32_TOL)])
def test_uneven_row_split_sum(dtype, tol):
    M, N, widths = 40, 512, (400, 600)
    K = sum(widths)
    log_case("uneven row split", M, N, widths, dtype)
    x, w, b = I.activations(M, K, 520, dtype=dtype), I.weight(N, K, 521, dtype=dtype), I.bias(N, 522, dtype=dtype)
    X, W, B = dev(x), dev(w), dev(b)
    parts, start = [], 0
    for width in widths:
        W_r = torch.empty(N, width, dtype=dtype, device="cuda")
        tp.tp_shard_weight_block(W, N, K, 1, start, width, W_r)
        P_r = torch.empty(M, N, dtype=dtype, device="cuda")
        tp.tp_linear_row_partial(X[:, start:], K, W_r, P_r, M, width, N, 1)  # this shard's input columns
        parts.append(P_r)
        start += width
    Y = torch.empty(M, N, dtype=dtype, device="cuda")
    tp.tp_combine_sum(parts, B, Y, M, N)
    torch.cuda.synchronize()
    assert err(Y, O.linear(host64(x), host64(w), host64(b))) <= tol


@pytest.mark.parametrize("M", [1, 64, 300])
def test_kv_heads_replicated_over_more_shards(M):
    """16 Q heads, 2 KV heads of 64, TP = 8: each KV head lives on 4 consecutive shards."""
    nh, nkv, d, hid, p = 16, 2, 64, 1024, 8
    log_case("kv replication", M, nh, nkv, d, p)
    shape = I.LayerShape("t", hidden=hid, n_heads=nh, n_kv_heads=nkv, head_dim=d, tp=p, seed=53)
    wt = I.attn_weights(shape)
    w64 = {k: host64(v) for k, v in wt.items()}
    x = I.activations(M, hid, 530 + M)
    a = I.activations(M, nh * d, 531 + M)
    X, A = dev(x), dev(a)
    Wqkv, Bqkv, Wo = dev(wt["Wqkv"]), dev(wt["bqkv"]), dev(wt["Wo"])
    hq = nh // p
    nq = (hq + 2) * d
    full = O.linear(host64(x), w64["Wqkv"], w64["bqkv"])
    parts = []
    for r in range(p):
        W_r = torch.empty(nq, hid, dtype=torch.bfloat16, device="cuda")
        b_r = torch.empty(nq, dtype=torch.bfloat16, device="cuda")
        tp.tp_shard_qkv(Wqkv, hid, nh, nkv, d, p, r, W_r)
        tp.tp_shard_qkv(Bqkv, 1, nh, nkv, d, p, r, b_r)
        Wo_r = torch.empty(hid, hq * d, dtype=torch.bfloat16, device="cuda")
        tp.tp_shard_weight(Wo, hid, nh * d, p, r, 1, Wo_r)
        QKV_r = torch.empty(M, nq, dtype=torch.bfloat16, device="cuda")
        P_r = torch.empty(M, hid, dtype=torch.bfloat16, device="cuda")
        tp.tp_attn_proj_shard(X, W_r, b_r, QKV_r, A[:, r * hq * d:(r + 1) * hq * d].contiguous(), Wo_r,
                              P_r, M, hid, nh, nkv, d, p)
        torch.cuda.synchronize()
        w_ref, b_ref = O.qkv_shard(w64["Wqkv"], w64["bqkv"], nh, nkv, d, p, r)
        np.testing.assert_array_equal(host64(W_r), w_ref)
        np.testing.assert_array_equal(host64(b_r), b_ref)
        h = O.kv_heads_of(nkv, p, r)[0]
        assert h == r * nkv // p
        y = host64(QKV_r)
        assert err(QKV_r, O.col_linear(host64(x), w_ref, b_ref)) <= BF16_TOL
        # its segments are Q of its own heads and a copy of the KV head it replicates
        np.testing.assert_allclose(y[:, hq * d:(hq + 1) * d], full[:, (nh + h) * d:(nh + h + 1) * d],
                                   atol=BF16_TOL * np.abs(full).max())
        parts.append(P_r)
    Y = torch.empty(M, hid, dtype=torch.bfloat16, device="cuda")
    tp.tp_combine_sum(parts, dev(wt["bo"]), Y, M, hid)
    torch.cuda.synchronize()
    assert err(Y, O.linear(host64(a), w64["Wo"], w64["bo"])) <= BF16_TOL
