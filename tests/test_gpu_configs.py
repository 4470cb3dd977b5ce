"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Every output element is compared with the fp64 oracle (numpy BLAS on the host makes the
whole 70B layer at 4096 tokens a matter of seconds): the large-tile prefill kernel's
256-token tiles are checked on every lane, wave and split-K piece, not on sampled rows."""
import numpy as np
import pytest
import torch

import oracle as O
import tensor_transformer_linear_col_amd as tp
import tp_inputs as I
from gpu_util import BF16_TOL, dev, err, host64, log_case

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def all_rows(M):
    return np.arange(M)


def shard_ffn_on_device(wt, p, inter, bias):
    """Per-shard device weights: column blocks of Wg/Wu (+ biases), input-column block of Wd."""
    Wg, Wu, Wd = dev(wt["Wg"]), dev(wt["Wu"]), dev(wt["Wd"])
    hidden = wt["Wd"].shape[0]
    i = inter // p
    out = []
    for r in range(p):
        s = {}
        for name, W in (("Wg", Wg), ("Wu", Wu)):
            s[name] = torch.empty(i, hidden, dtype=BF, device="cuda")
            tp.tp_shard_weight(W, inter, hidden, p, r, 0, s[name])
        s["Wd"] = torch.empty(hidden, i, dtype=BF, device="cuda")
        tp.tp_shard_weight(Wd, hidden, inter, p, r, 1, s["Wd"])
        for name in ("bg", "bu"):
            if bias:
                s[name] = torch.empty(i, dtype=BF, device="cuda")
                tp.tp_shard_weight(dev(wt[name]), inter, 1, p, r, 0, s[name])
            else:
                s[name] = None
        out.append(s)
    del Wg, Wu, Wd
    return out


def run_mlp(X, shards, M, hidden, inter, p, bd):
    i = inter // p
    parts, hs = [], []
    for r, s in enumerate(shards):
        H_r = torch.empty(M, i, dtype=BF, device="cuda")
        P_r = torch.empty(M, hidden, dtype=BF, device="cuda")
        tp.tp_mlp_shard(X, s["Wg"], s["Wu"], s["bg"], s["bu"], s["Wd"], H_r, P_r, M, hidden, inter, p)
        parts.append(P_r)
        hs.append(H_r)
    Y = torch.empty(M, hidden, dtype=BF, device="cuda")
    tp.tp_combine_sum(parts, bd, Y, M, hidden)
    H = torch.empty(M, inter, dtype=BF, device="cuda")
    tp.tp_combine_concat(hs, [i], H, M)
    torch.cuda.synchronize()
    return Y, H, parts


def check_ffn(shape, M, bias):
    log_case("ffn config", shape.name, M, bias)
    h, inter, p = shape.hidden, shape.intermediate, shape.tp
    wt = I.ffn_weights(shape, with_bias=bias)
    x = I.activations(M, h, I.activation_seed(shape.seed, M))
    shards = shard_ffn_on_device(wt, p, inter, bias)
    Y, H, _ = run_mlp(dev(x), shards, M, h, inter, p, dev(wt["bd"]) if bias else None)
    rows = all_rows(M)
    xs = host64(x)[rows]
    w64 = {k: host64(v) for k, v in wt.items()}
    h_ref = O.swiglu(O.linear(xs, w64["Wg"], w64.get("bg")), O.linear(xs, w64["Wu"], w64.get("bu")))
    y_ref = O.linear(h_ref, w64["Wd"], w64.get("bd"))
    assert err(H.cpu()[rows], h_ref) <= BF16_TOL
    assert err(Y.cpu()[rows], y_ref) <= BF16_TOL


@pytest.mark.parametrize("M", [1, 8, 64])
def test_llama7b_ffn_tp2(M):
    check_ffn(I.LLAMA7B_FFN_TP2, M, bias=False)


def test_llama7b_ffn_tp2_with_bias():
    check_ffn(I.LLAMA7B_FFN_TP2, 8, bias=True)


@pytest.mark.parametrize("M", [1, 16, 64])
def test_llama70b_ffn_tp4(M):
    check_ffn(I.LLAMA70B_FFN_TP4, M, bias=False)


@pytest.mark.parametrize("M", [1, 2048])
def test_llama70b_attn_proj_tp8(M):
    shape = I.LLAMA70B_ATTN_TP8
    log_case("attn config", shape.name, M)
    h, nh, nkv, d, p = shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.tp
    wt = I.attn_weights(shape, with_bias=False)
    x = I.activations(M, h, I.activation_seed(shape.seed, M))
    a = I.activations(M, nh * d, I.activation_seed(shape.seed, M, slot=1))
    Wqkv, Wo = dev(wt["Wqkv"]), dev(wt["Wo"])
    X, A = dev(x), dev(a)
    nq, ka = (nh // p + 2 * nkv // p) * d, nh // p * d
    qkvs, parts = [], []
    for r in range(p):
        W_r = torch.empty(nq, h, dtype=BF, device="cuda")
        Wo_r = torch.empty(h, ka, dtype=BF, device="cuda")
        tp.tp_shard_qkv(Wqkv, h, nh, nkv, d, p, r, W_r)
        tp.tp_shard_weight(Wo, h, nh * d, p, r, 1, Wo_r)
        QKV_r = torch.empty(M, nq, dtype=BF, device="cuda")
        P_r = torch.empty(M, h, dtype=BF, device="cuda")
        tp.tp_attn_proj_shard(X, W_r, None, QKV_r, A[:, r * ka:(r + 1) * ka].contiguous(), Wo_r, P_r,
                              M, h, nh, nkv, d, p)
        qkvs.append(QKV_r)
        parts.append(P_r)
    QKV = torch.empty(M, (nh + 2 * nkv) * d, dtype=BF, device="cuda")
    tp.tp_combine_concat(qkvs, list(O.qkv_segments(nh, nkv, d, p)), QKV, M)
    Y = torch.empty(M, h, dtype=BF, device="cuda")
    tp.tp_combine_sum(parts, None, Y, M, h)
    torch.cuda.synchronize()
    rows = all_rows(M)
    assert err(QKV.cpu()[rows], O.linear(host64(x)[rows], host64(wt["Wqkv"]))) <= BF16_TOL
    assert err(Y.cpu()[rows], O.linear(host64(a)[rows], host64(wt["Wo"]))) <= BF16_TOL
    # per-shard outputs, every row, against the oracle's own shards
    for r in (0, p - 1):
        w_ref, _ = O.qkv_shard(host64(wt["Wqkv"]), None, nh, nkv, d, p, r)
        assert err(qkvs[r].cpu()[rows], O.col_linear(host64(x)[rows], w_ref)) <= BF16_TOL


def test_llama70b_layer_prefill_tp8():
    """The whole layer: 8 shards looped on the device, combined on the device, checked
    against the unsharded fp64 chain on every token row; H (the gate/up + SwiGLU output of
    every shard) against the oracle on the device's own Y1."""
    shape = I.LLAMA70B_LAYER_TP8
    M = shape.tokens[0]
    log_case("layer config", shape.name, M)
    h, inter, nh, nkv, d, p = (shape.hidden, shape.intermediate, shape.n_heads, shape.n_kv_heads,
                               shape.head_dim, shape.tp)
    aw = I.attn_weights(shape, with_bias=True)
    fw = I.ffn_weights(shape, with_bias=True)
    x = I.activations(M, h, I.activation_seed(shape.seed, M))
    X = dev(x)
    nq, ka = (nh // p + 2 * nkv // p) * d, nh // p * d
    Wqkv, bqkv, Wo = dev(aw["Wqkv"]), dev(aw["bqkv"]), dev(aw["Wo"])
    qkvs, o_parts = [], []
    for r in range(p):
        W_r = torch.empty(nq, h, dtype=BF, device="cuda")
        b_r = torch.empty(nq, dtype=BF, device="cuda")
        Wo_r = torch.empty(h, ka, dtype=BF, device="cuda")
        tp.tp_shard_qkv(Wqkv, h, nh, nkv, d, p, r, W_r)
        tp.tp_shard_qkv(bqkv, 1, nh, nkv, d, p, r, b_r)
        tp.tp_shard_weight(Wo, h, nh * d, p, r, 1, Wo_r)
        QKV_r = torch.empty(M, nq, dtype=BF, device="cuda")
        tp.tp_attn_proj_shard(X, W_r, b_r, QKV_r, None, None, None, M, h, nh, nkv, d, p)
        P_r = torch.empty(M, h, dtype=BF, device="cuda")
        # A := Q, the shard's own heads: the first ka columns of QKV_r (row stride nq)
        tp.tp_linear_row_partial(QKV_r, nq, Wo_r, P_r, M, nh * d, h, p)
        qkvs.append(QKV_r)
        o_parts.append(P_r)
    del Wqkv, Wo
    Y1 = torch.empty(M, h, dtype=BF, device="cuda")
    tp.tp_combine_sum(o_parts, dev(aw["bo"]), Y1, M, h)
    QKV = torch.empty(M, (nh + 2 * nkv) * d, dtype=BF, device="cuda")
    tp.tp_combine_concat(qkvs, list(O.qkv_segments(nh, nkv, d, p)), QKV, M)
    del o_parts
    shards = shard_ffn_on_device(fw, p, inter, True)
    Y, H, _ = run_mlp(Y1, shards, M, h, inter, p, dev(fw["bd"]))
    rows = all_rows(M)
    w = {k: host64(v) for k, v in {**aw, **fw}.items()}
    w.update(n_heads=nh, n_kv_heads=nkv, head_dim=d)
    xs = host64(x)[rows]
    y_ref = O.layer_unsharded(xs, w)
    qkv_ref = O.linear(xs, w["Wqkv"], w["bqkv"])
    assert err(QKV.cpu()[rows], qkv_ref) <= BF16_TOL
    y1_ref = O.linear(qkv_ref[:, :nh * d], w["Wo"], w["bo"])
    assert err(Y1.cpu()[rows], y1_ref) <= BF16_TOL
    assert err(Y.cpu()[rows], y_ref) <= BF16_TOL
    # The gate/up + SwiGLU output of every shard (the concat of the H_r), against the oracle
    # on exactly that product's inputs (the device's Y1).
    y1_dev = host64(Y1.cpu())
    h_ref = O.swiglu(O.linear(y1_dev, w["Wg"], w["bg"]), O.linear(y1_dev, w["Wu"], w["bu"]))
    assert err(H.cpu(), h_ref) <= BF16_TOL
