"""GPU parity of every entry point against the fp64 oracle, at sizes the oracle finishes
in seconds that still span several tiles, ragged tails and the degenerate cases.
Every call goes through the C ABI (the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle as O
import tensor_transformer_linear_col_amd as tp
import tp_inputs as I
from conftest import read_golden
from gpu_util import (BF16_TOL, F32_TOL, canaries_intact, canary_buffer, dev, err, host64,
                      log_case)

pytestmark = pytest.mark.gpu


# ---- the toy layer: fp32, TP = 2 ("Tensor parallel serving", simulation script) ------------

def test_toy_column_split_concat_fp32():
    log_case("toy column split fp32")
    x, w, b = I.toy_layer()
    X, W, B = dev(x), dev(w), dev(b)
    shards = []
    for r in range(2):
        W_r = torch.empty(3, 8, device="cuda")
        b_r = torch.empty(3, device="cuda")
        tp.tp_shard_weight(W, 6, 8, 2, r, 0, W_r)
        tp.tp_shard_weight(B, 6, 1, 2, r, 0, b_r)
        Y_r = torch.empty(1, 3, device="cuda")
        tp.tp_linear_col(X, W_r, b_r, Y_r, 1, 8, 6, 2)
        shards.append(Y_r)
    Y = torch.empty(1, 6, device="cuda")
    tp.tp_combine_concat(shards, [3], Y, 1)
    torch.cuda.synchronize()
    ref = O.linear(host64(x), host64(w), host64(b))
    assert err(Y, ref) <= F32_TOL
    printed = [float(v) for v in read_golden("toy_tp2.txt")["combined_output_round4"]]
    np.testing.assert_array_equal(np.round(host64(Y)[0], 4), printed)
    assert W_r.numel() == 24   # the printed output's weight count of one shard: 24 of the 48


def test_toy_row_split_sum_fp32():
    log_case("toy row split fp32")
    x, w, b = I.toy_layer()
    X, W, B = dev(x), dev(w), dev(b)
    parts = []
    for r in range(2):
        W_r = torch.empty(6, 4, device="cuda")
        tp.tp_shard_weight(W, 6, 8, 2, r, 1, W_r)
        P_r = torch.empty(1, 6, device="cuda")
        tp.tp_linear_row_partial(X[:, r * 4:], 8, W_r, P_r, 1, 8, 6, 2)   # the rank's slice of x
        parts.append(P_r)
    Y = torch.empty(1, 6, device="cuda")
    tp.tp_combine_sum(parts, B, Y, 1, 6)
    torch.cuda.synchronize()
    ref = O.linear(host64(x), host64(w), host64(b))
    assert err(Y, ref) <= F32_TOL
    printed = [float(v) for v in read_golden("toy_tp2.txt")["full_output_round4"]]
    np.testing.assert_array_equal(np.round(host64(Y)[0], 4), printed)


# ---- bf16 column linear: decode kernel (M <= 64) and prefill kernel (M > 64) -----------------

SHAPES = [  # (M, K, N): ragged M, K and N tails, several tiles, both kernels
    (1, 8, 16), (1, 40, 3), (1, 4096, 1280), (2, 1000, 200), (5, 520, 24), (8, 4096, 344),
    (16, 264, 48), (17, 1032, 100), (33, 2048, 130), (48, 96, 64), (64, 4104, 200), (65, 512, 96),
    (100, 1000, 300), (130, 264, 257), (256, 1024, 512), (300, 2056, 520), (513, 640, 264),
]


@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_linear_col_bf16(M, K, N, bias):
    log_case("linear_col bf16", M, K, N, bias)
    seed = M * 7 + K * 3 + N
    x = I.activations(M, K, seed)
    w = I.weight(N, K, seed + 1)
    b = I.bias(N, seed + 2) if bias else None
    buf, Y = canary_buffer((M, N), torch.bfloat16)
    tp.tp_linear_col(dev(x), dev(w), dev(b), Y, M, K, N, 1)
    torch.cuda.synchronize()
    ref = O.linear(host64(x), host64(w), None if b is None else host64(b))
    assert err(Y, ref) <= BF16_TOL
    assert canaries_intact(buf, (M, N))


@pytest.mark.parametrize("M,K,N", [(1, 4096, 1280), (9, 4096, 1280), (16, 1000, 8200), (37, 2048, 96),
                                   (64, 2056, 520), (300, 1024, 264)])
def test_linear_col_bf16_fp32_partial_out(M, K, N):
    """bf16 inputs with fp32 outputs (the row layer's fp32-partial option) are tighter."""
    log_case("row partial fp32 out", M, K, N)
    x, w = I.activations(M, K, 5), I.weight(N, K, 6)
    P = torch.empty(M, N, device="cuda", dtype=torch.float32)
    tp.tp_linear_row_partial(dev(x), K, dev(w), P, M, K, N, 1)
    torch.cuda.synchronize()
    assert err(P, O.linear(host64(x), host64(w))) <= 1e-5


@pytest.mark.parametrize("M", [1, 3, 64, 200])
@pytest.mark.parametrize("p", [2, 4])
def test_row_partial_rank_slices_sum(M, p):
    """Row split with the rank's slice of a full X (ldx = K) and the bias added once."""
    log_case("row split sum", M, p)
    K, N = 1024, 320
    x, w, b = I.activations(M, K, 11), I.weight(N, K, 12), I.bias(N, 13)
    X, W = dev(x), dev(w)
    parts = []
    for r in range(p):
        W_r = torch.empty(N, K // p, dtype=torch.bfloat16, device="cuda")
        tp.tp_shard_weight(W, N, K, p, r, 1, W_r)
        P_r = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        tp.tp_linear_row_partial(X[:, r * (K // p):], K, W_r, P_r, M, K, N, p)
        parts.append(P_r)
        ref_r = O.row_partial(O.input_slice(host64(x), p, r), O.row_shard(host64(w), p, r))
        torch.cuda.synchronize()
        assert err(P_r, ref_r) <= BF16_TOL
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tp.tp_combine_sum(parts, dev(b), Y, M, N)
    torch.cuda.synchronize()
    assert err(Y, O.linear(host64(x), host64(w), host64(b))) <= BF16_TOL


# ---- SwiGLU MLP shard -------------------------------------------------------------------------

@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("M", [1, 7, 16, 40, 64, 65, 300])
def test_mlp_shard_bf16(M, bias):
    log_case("mlp shard", M, bias)
    h, inter, p = 1024, 3072, 2
    shape = I.LayerShape("t", hidden=h, intermediate=inter, tp=p, seed=40 + M)
    wt = I.ffn_weights(shape, with_bias=bias)
    x = I.activations(M, h, 41 + M)
    X = dev(x)
    parts = []
    hs = []
    for r in range(p):
        Wg_r, bg_r = O.col_shard(host64(wt["Wg"]), host64(wt["bg"]) if bias else None, p, r)
        i = inter // p
        sl = slice(r * i, (r + 1) * i)
        H_r = torch.empty(M, i, dtype=torch.bfloat16, device="cuda")
        P_r = torch.empty(M, h, dtype=torch.bfloat16, device="cuda")
        tp.tp_mlp_shard(X, dev(wt["Wg"][sl]), dev(wt["Wu"][sl]),
                        dev(wt["bg"][sl]) if bias else None, dev(wt["bu"][sl]) if bias else None,
                        dev(wt["Wd"][:, sl]), H_r, P_r, M, h, inter, p)
        torch.cuda.synchronize()
        h_ref, p_ref = O.mlp_shard(host64(x), Wg_r, host64(wt["Wu"][sl]), host64(wt["Wd"][:, sl]),
                                   bg_r, host64(wt["bu"][sl]) if bias else None)
        assert err(H_r, h_ref) <= BF16_TOL
        # the partial is checked against the oracle applied to the GPU's own bf16 H_r
        assert err(P_r, O.row_partial(host64(H_r), host64(wt["Wd"][:, sl]))) <= BF16_TOL
        assert err(P_r, p_ref) <= BF16_TOL
        parts.append(P_r)
        hs.append(H_r)
    Y = torch.empty(M, h, dtype=torch.bfloat16, device="cuda")
    tp.tp_combine_sum(parts, dev(wt["bd"]) if bias else None, Y, M, h)
    Hc = torch.empty(M, inter, dtype=torch.bfloat16, device="cuda")
    tp.tp_combine_concat(hs, [inter // p], Hc, M)
    torch.cuda.synchronize()
    w64 = {k: host64(v) for k, v in wt.items()}
    ref = O.mlp(host64(x), w64["Wg"], w64["Wu"], w64["Wd"], w64.get("bg"), w64.get("bu"), w64.get("bd"))
    assert err(Y, ref) <= BF16_TOL
    h_full = O.swiglu(O.linear(host64(x), w64["Wg"], w64.get("bg")), O.linear(host64(x), w64["Wu"], w64.get("bu")))
    assert err(Hc, h_full) <= BF16_TOL


def test_mlp_shard_fp32_and_skip_down():
    log_case("mlp shard fp32")
    M, h, inter, p = 5, 64, 96, 2
    shape = I.LayerShape("t", hidden=h, intermediate=inter, tp=p, seed=50)
    wt = I.ffn_weights(shape, dtype=torch.float32)
    x = I.activations(M, h, 51, dtype=torch.float32)
    i = inter // p
    H_r = torch.empty(M, i, device="cuda")
    tp.tp_mlp_shard(dev(x), dev(wt["Wg"][:i]), dev(wt["Wu"][:i]), dev(wt["bg"][:i]), dev(wt["bu"][:i]),
                    None, H_r, None, M, h, inter, p)
    torch.cuda.synchronize()
    w64 = {k: host64(v) for k, v in wt.items()}
    ref = O.swiglu(O.linear(host64(x), w64["Wg"][:i], w64["bg"][:i]), O.linear(host64(x), w64["Wu"][:i], w64["bu"][:i]))
    assert err(H_r, ref) <= F32_TOL


# ---- decode tile choices: SwiGLU pair with two gate + two up tiles per wave and whole K (3-32
# tokens, where the 32-output row groups fill the chip), three token tiles run as four (33-48
# tokens), plain products with two row tiles (from 5 tokens), equal ranges per CU for long SwiGLU
# weight streams (1-2 tokens, or more where the 2 + 2 row groups do not fill the chip); ragged
# output counts, K tails, bias, bitwise reproducibility.

@pytest.mark.parametrize("M,K,I_,bias", [(3, 1000, 6600, True), (9, 4096, 7168, False),
                                         (16, 8192, 7176, True), (2, 1000, 6600, False),
                                         (20, 2056, 6600, True), (32, 4096, 7176, False),
                                         (40, 1000, 6600, True), (48, 2048, 1000, False),
                                         (1, 8192, 7176, True), (2, 6000, 7000, False),
                                         (12, 16384, 4104, True)])
def test_decode_swiglu_wide_tiles(M, K, I_, bias):
    log_case("decode swiglu wide tiles", M, K, I_, bias)
    wg, wu = I.weight(I_, K, 60 + M), I.weight(I_, K, 61 + M)
    bg, bu = (I.bias(I_, 62), I.bias(I_, 63)) if bias else (None, None)
    x = I.activations(M, K, 64 + M)
    X, Wg, Wu, Bg, Bu = dev(x), dev(wg), dev(wu), dev(bg), dev(bu)
    buf, H = canary_buffer((M, I_), torch.bfloat16)
    tp.tp_mlp_shard(X, Wg, Wu, Bg, Bu, None, H, None, M, K, I_, 1)
    H2 = torch.empty(M, I_, dtype=torch.bfloat16, device="cuda")
    tp.tp_mlp_shard(X, Wg, Wu, Bg, Bu, None, H2, None, M, K, I_, 1)
    torch.cuda.synchronize()
    ref = O.swiglu(O.linear(host64(x), host64(wg), None if bg is None else host64(bg)),
                   O.linear(host64(x), host64(wu), None if bu is None else host64(bu)))
    assert err(H, ref) <= BF16_TOL
    assert canaries_intact(buf, (M, I_))
    assert torch.equal(H, H2)


@pytest.mark.parametrize("M,K,N,bias", [(5, 1000, 8200, True), (12, 7000, 8192, False), (16, 4096, 4104, True),
                                        (4, 1000, 8200, False)])
def test_decode_plain_two_tiles(M, K, N, bias):
    log_case("decode plain two tiles", M, K, N, bias)
    x, w = I.activations(M, K, 70 + M), I.weight(N, K, 71 + M)
    b = I.bias(N, 72) if bias else None
    X, W, B = dev(x), dev(w), dev(b)
    buf, Y = canary_buffer((M, N), torch.bfloat16)
    tp.tp_linear_col(X, W, B, Y, M, K, N, 1)
    Y2 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tp.tp_linear_col(X, W, B, Y2, M, K, N, 1)
    torch.cuda.synchronize()
    assert err(Y, O.linear(host64(x), host64(w), None if b is None else host64(b))) <= BF16_TOL
    assert canaries_intact(buf, (M, N))
    assert torch.equal(Y, Y2)


# ---- head-split attention projections ----------------------------------------------------------

@pytest.mark.parametrize("M", [1, 9, 130])
def test_attn_proj_shards_and_combines(M):
    log_case("attn proj", M)
    nh, nkv, d, h, p = 16, 4, 32, 512, 4
    shape = I.LayerShape("t", hidden=h, n_heads=nh, n_kv_heads=nkv, head_dim=d, tp=p, seed=60 + M)
    wt = I.attn_weights(shape)
    x = I.activations(M, h, 61 + M)
    a_full = I.activations(M, nh * d, 62 + M)
    Wqkv, bqkv, Wo = dev(wt["Wqkv"]), dev(wt["bqkv"]), dev(wt["Wo"])
    nq = (nh // p + 2 * nkv // p) * d
    ka = nh // p * d
    qkvs, parts = [], []
    for r in range(p):
        W_r = torch.empty(nq, h, dtype=torch.bfloat16, device="cuda")
        b_r = torch.empty(nq, dtype=torch.bfloat16, device="cuda")
        Wo_r = torch.empty(h, ka, dtype=torch.bfloat16, device="cuda")
        tp.tp_shard_qkv(Wqkv, h, nh, nkv, d, p, r, W_r)
        tp.tp_shard_qkv(bqkv, 1, nh, nkv, d, p, r, b_r)
        tp.tp_shard_weight(Wo, h, nh * d, p, r, 1, Wo_r)
        QKV_r = torch.empty(M, nq, dtype=torch.bfloat16, device="cuda")
        P_r = torch.empty(M, h, dtype=torch.bfloat16, device="cuda")
        A_r = dev(a_full[:, r * ka:(r + 1) * ka])
        tp.tp_attn_proj_shard(dev(x), W_r, b_r, QKV_r, A_r, Wo_r, P_r, M, h, nh, nkv, d, p)
        torch.cuda.synchronize()
        w_ref, b_ref = O.qkv_shard(host64(wt["Wqkv"]), host64(wt["bqkv"]), nh, nkv, d, p, r)
        np.testing.assert_array_equal(host64(W_r), w_ref)   # the head split itself is exact
        np.testing.assert_array_equal(host64(b_r), b_ref)
        assert err(QKV_r, O.col_linear(host64(x), w_ref, b_ref)) <= BF16_TOL
        assert err(P_r, O.row_partial(host64(a_full)[:, r * ka:(r + 1) * ka], O.row_shard(host64(wt["Wo"]), p, r))) <= BF16_TOL
        qkvs.append(QKV_r)
        parts.append(P_r)
    QKV = torch.empty(M, (nh + 2 * nkv) * d, dtype=torch.bfloat16, device="cuda")
    seg = O.qkv_segments(nh, nkv, d, p)
    tp.tp_combine_concat(qkvs, list(seg), QKV, M)
    Y = torch.empty(M, h, dtype=torch.bfloat16, device="cuda")
    tp.tp_combine_sum(parts, dev(wt["bo"]), Y, M, h)
    torch.cuda.synchronize()
    assert err(QKV, O.linear(host64(x), host64(wt["Wqkv"]), host64(wt["bqkv"]))) <= BF16_TOL
    assert err(Y, O.linear(host64(a_full), host64(wt["Wo"]), host64(wt["bo"]))) <= BF16_TOL
    # concat is a pure copy: bit-exact against the oracle's segment concat of the GPU shards
    np.testing.assert_array_equal(host64(QKV), O.concat([host64(q) for q in qkvs], seg))


# ---- combines: exactness, dtypes, ragged sizes ---------------------------------------------

@pytest.mark.parametrize("pdt,odt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.bfloat16),
                                     (torch.float32, torch.float32), (torch.bfloat16, torch.float32)])
@pytest.mark.parametrize("M,N,p", [(1, 8, 2), (3, 13, 3), (7, 4096, 8), (5, 1000, 4)])
def test_combine_sum(M, N, p, pdt, odt):
    log_case("combine sum", M, N, p, pdt, odt)
    parts = [I.activations(M, N, 70 + r, dtype=torch.float32).to(pdt) for r in range(p)]
    b = I.bias(N, 79, dtype=torch.float32).to(odt)
    Y = torch.empty(M, N, dtype=odt, device="cuda")
    tp.tp_combine_sum([dev(t) for t in parts], dev(b), Y, M, N)
    torch.cuda.synchronize()
    ref = O.combine_sum([host64(t) for t in parts], host64(b))
    tol = BF16_TOL if odt == torch.bfloat16 else 1e-6
    assert err(Y, ref) <= tol
    # the same fp32 accumulation order on the host gives the identical fp32 result
    if odt == torch.float32:
        acc = torch.zeros(M, N, dtype=torch.float32)
        for t in parts:
            acc = acc + t.float()
        acc = acc + b.float()
        assert torch.equal(acc, Y.cpu())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,segs,p", [(1, [3], 2), (4, [5, 4], 2), (6, [1024, 128, 128], 8), (3, [7], 3)])
def test_combine_concat_exact(M, segs, p, dtype):
    log_case("concat", M, segs, p, dtype)
    s = sum(segs)
    shards = [I.activations(M, s, 90 + r, dtype=torch.float32).to(dtype) for r in range(p)]
    Y = torch.empty(M, p * s, dtype=dtype, device="cuda")
    tp.tp_combine_concat([dev(t) for t in shards], segs, Y, M)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host64(Y), O.concat([host64(t) for t in shards], segs))


def test_uneven_split_five_plus_four_via_concat():
    """'Try it yourself' on the GPU: 9 outputs as shards of 5 and 4, each computed as a
    column product, then concatenated (the ABI's even split is bypassed with p = 1 calls)."""
    log_case("uneven 5+4")
    x, w, b = I.toy_layer_uneven(9)
    X = dev(x)
    outs = []
    for lo, hi in ((0, 5), (5, 9)):
        Y_r = torch.empty(1, hi - lo, device="cuda")
        tp.tp_linear_col(X, dev(w[lo:hi]), dev(b[lo:hi]), Y_r, 1, 8, hi - lo, 1)
        outs.append(Y_r)
    torch.cuda.synchronize()
    got = np.concatenate([host64(o) for o in outs], axis=-1)
    assert O.rel_err(got, O.linear(host64(x), host64(w), host64(b))) <= F32_TOL


def test_shard_weight_exact():
    log_case("shard weight")
    w = I.weight(48, 40, 99)
    W = dev(w)
    for p in (1, 2, 4, 8):
        for r in range(p):
            c = torch.empty(48 // p, 40, dtype=torch.bfloat16, device="cuda")
            tp.tp_shard_weight(W, 48, 40, p, r, 0, c)
            rr = torch.empty(48, 40 // p if 40 % p == 0 else 1, dtype=torch.bfloat16, device="cuda")
            if 40 % p == 0:
                tp.tp_shard_weight(W, 48, 40, p, r, 1, rr)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(host64(c), O.col_shard(host64(w), None, p, r)[0])
            if 40 % p == 0:
                np.testing.assert_array_equal(host64(rr), O.row_shard(host64(w), p, r))


# ---- determinism, M = 0, error path on the device ------------------------------------------

@pytest.mark.parametrize("M,K,N", [(1, 8192, 1280), (64, 4096, 688), (300, 2048, 520), (1000, 16384, 1320)])
def test_bitwise_deterministic(M, K, N):
    log_case("deterministic", M, K, N)
    x, w, b = I.activations(M, K, 1), I.weight(N, K, 2), I.bias(N, 3)
    X, W, B = dev(x), dev(w), dev(b)
    Y1 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Y2 = torch.empty_like(Y1)
    tp.tp_linear_col(X, W, B, Y1, M, K, N, 1)
    tp.tp_linear_col(X, W, B, Y2, M, K, N, 1)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


def test_zero_tokens_is_a_no_op():
    Y = torch.full((4, 16), 7.0, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(16, 8, dtype=torch.bfloat16, device="cuda")
    X = torch.zeros(1, 8, dtype=torch.bfloat16, device="cuda")
    tp.tp_linear_col(X, W, None, Y, 0, 8, 16, 1)
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())


def test_errors_raise_before_launch():
    X = torch.zeros(2, 4096, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(11008 // 2, 4096, dtype=torch.bfloat16, device="cuda")
    Y = torch.zeros(2, 11008 // 2, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tp.TPError) as e:
        tp.tp_linear_col(X, W, None, Y, 2, 4096, 11008, 3)
    assert e.value.status == 3


# ---- the large-tile LDS-DMA kernel: ragged token and feature tails ------------------------
# It runs when 256 x 256 tiles (128 x 256 for SwiGLU) alone fill the chip and K is a
# multiple of 64, so these shapes are large; the oracle checks every token row.

DMA_SHAPES = [  # (M, K, N): tails in M and N, K a multiple of 64
    (2100, 1024, 8168), (4096 + 33, 576, 8192 - 40), (8192, 128, 8192 + 8),
    (4096 - 40, 1024, 8192 - 24),  # 512 tiles: one tile per workgroup, ragged edges
    (4096, 256, 8190),  # output rows not a whole number of 16-byte runs: per-element stores
]


def _sample_rows(M):
    """Every token row (the name is kept for the tests below)."""
    return np.arange(M)


@pytest.mark.parametrize("M,K,N", DMA_SHAPES)
def test_dma_kernel_tails(M, K, N):
    log_case("dma kernel tails", M, K, N)
    x, w, b = I.activations(M, K, 301), I.weight(N, K, 302), I.bias(N, 303)
    buf, Y = canary_buffer((M, N), torch.bfloat16)
    tp.tp_linear_col(dev(x), dev(w), dev(b), Y, M, K, N, 1)
    torch.cuda.synchronize()
    rows = _sample_rows(M)
    ref = O.linear(host64(x)[rows], host64(w), host64(b))
    assert err(Y.cpu()[rows], ref) <= BF16_TOL
    assert canaries_intact(buf, (M, N))


@pytest.mark.parametrize("M,K,I_", [(2310, 512, 3584 - 24), (4096, 64, 4096 + 40)])
def test_dma_kernel_swiglu_tails(M, K, I_):
    log_case("dma kernel swiglu tails", M, K, I_)
    x = I.activations(M, K, 311)
    wg, wu = I.weight(I_, K, 312), I.weight(I_, K, 313)
    bg, bu = I.bias(I_, 314), I.bias(I_, 315)
    buf, H = canary_buffer((M, I_), torch.bfloat16)
    tp.tp_mlp_shard(dev(x), dev(wg), dev(wu), dev(bg), dev(bu), None, H, None, M, K, I_, 1)
    torch.cuda.synchronize()
    rows = _sample_rows(M)
    xs = host64(x)[rows]
    ref = O.swiglu(O.linear(xs, host64(wg), host64(bg)), O.linear(xs, host64(wu), host64(bu)))
    assert err(H.cpu()[rows], ref) <= BF16_TOL
    assert canaries_intact(buf, (M, I_))


# 160 x 128 tiles on 16-row MFMA blocks: plain products with fewer 256 x 256 tiles than CUs
# whose 160 x 128 tiles fill whole waves (the 70B TP=8 QKV shard's 1280 x 4096 outputs are 256
# tiles), or fewer, each cut into the K ranges that fill the chip (1280 x 2048: 2; 1280 x 1024: 4;
# 1280 x 256: 16; 1270 x 768: 5); ragged features and tokens, bias or none, bf16 output or an fp32
# row partial.
@pytest.mark.parametrize("M,K,N,bias,f32", [(4096, 8192, 1280, True, False), (4000, 4096, 1250, True, False),
                                            (3900, 2048, 2552, False, False), (4096, 2048, 1280, False, True),
                                            (2000, 4096, 1250, True, False), (2048, 2048, 1280, False, True),
                                            (256, 8192, 1280, True, False), (768, 4096, 1270, False, False),
                                            (512, 2048, 2560, True, False), (1024, 4096, 1280, False, True)])
def test_dtl16_tiles(M, K, N, bias, f32):
    log_case("160x128 tiles on 16-row MFMA blocks", M, K, N, bias, f32)
    x, w = I.activations(M, K, 361), I.weight(N, K, 362)
    b = I.bias(N, 363) if bias else None
    buf, Y = canary_buffer((M, N), torch.float32 if f32 else torch.bfloat16)
    if f32:
        tp.tp_linear_row_partial(dev(x), K, dev(w), Y, M, K, N, 1)
    else:
        tp.tp_linear_col(dev(x), dev(w), dev(b), Y, M, K, N, 1)
    torch.cuda.synchronize()
    ref = O.linear(host64(x), host64(w), None if b is None else host64(b))
    assert err(Y.cpu(), ref) <= BF16_TOL
    assert canaries_intact(buf, (M, N))


# 21-64 tokens of a plain product (K >= 2048, a multiple of 64): one 64-token tile of 128 features per
# piece on 16-row MFMA blocks, each tile's K cut into S ranges (S = 8 for the 7B TP=2 down shard
# and for 3 tiles, 4 for the 70B TP=4 one, 2 for 100 tiles, 1 for 157), fp32 partials summed in K
# order by the reduce pass.
@pytest.mark.parametrize("M,K,N,bias,f32", [(64, 5504, 4096, False, False), (64, 7168, 8192, False, True),
                                            (40, 2048, 12800, True, False), (33, 2048, 300, True, False),
                                            (50, 4096, 20000, False, False), (48, 2048, 1300, False, True),
                                            (48, 2048, 1300, True, False), (21, 4096, 3000, True, False),
                                            (32, 7168, 8192, False, True)])
def test_dtl16_decode_split(M, K, N, bias, f32):
    assert not (bias and f32), "the row partial has no bias"
    log_case("21-64 tokens on 16-row MFMA blocks, split K", M, K, N, bias, f32)
    x, w = I.activations(M, K, 371), I.weight(N, K, 372)
    b = I.bias(N, 373) if bias else None
    buf, Y = canary_buffer((M, N), torch.float32 if f32 else torch.bfloat16)
    if f32:
        tp.tp_linear_row_partial(dev(x), K, dev(w), Y, M, K, N, 1)
    else:
        tp.tp_linear_col(dev(x), dev(w), dev(b), Y, M, K, N, 1)
    torch.cuda.synchronize()
    ref = O.linear(host64(x), host64(w), None if b is None else host64(b))
    assert err(Y.cpu(), ref) <= BF16_TOL
    assert canaries_intact(buf, (M, N))
    # bitwise repeatable: the K ranges are summed in a fixed order
    Y2 = torch.empty_like(Y)
    if f32:
        tp.tp_linear_row_partial(dev(x), K, dev(w), Y2, M, K, N, 1)
    else:
        tp.tp_linear_col(dev(x), dev(w), dev(b), Y2, M, K, N, 1)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)


# The SwiGLU pair on the same path (17-64 tokens; fewer below): 64 pairs x 64 tokens per piece, gate and up blocks of the
# same pairs in every wave (the 7B TP=2 and 70B TP=4 gate/up shards at 64 tokens, ragged pairs,
# one K range when the tiles alone fill the chip); 17-48 tokens with 205-256 tiles of 32 pairs
# (the 70B shard, 8000 pairs), whole-K tiles of 32 pairs in a 10-deep ring; and the same shapes
# below 17 tokens, which stay on the decode kernel.
@pytest.mark.parametrize("M,K,I_,bias", [(64, 4096, 5504, False), (64, 8192, 7168, True), (33, 2048, 1000, True),
                                         (48, 4096, 3000, False), (60, 2048, 20000, True), (17, 8192, 7168, False),
                                         (24, 4096, 5504, True), (32, 8192, 7168, True), (48, 4096, 8000, False),
                                         (1, 8192, 7168, True), (4, 8192, 7000, False), (8, 4096, 8192, True),
                                         (16, 2048, 6600, False)])
def test_dtl16_decode_swiglu(M, K, I_, bias):
    log_case("17-64 tokens SwiGLU on 16-row MFMA blocks, split K", M, K, I_, bias)
    x = I.activations(M, K, 381)
    wg, wu = I.weight(I_, K, 382), I.weight(I_, K, 383)
    bg, bu = (I.bias(I_, 384), I.bias(I_, 385)) if bias else (None, None)
    buf, H = canary_buffer((M, I_), torch.bfloat16)
    tp.tp_mlp_shard(dev(x), dev(wg), dev(wu), dev(bg), dev(bu), None, H, None, M, K, I_, 1)
    torch.cuda.synchronize()
    xs = host64(x)
    ref = O.swiglu(O.linear(xs, host64(wg), None if bg is None else host64(bg)),
                   O.linear(xs, host64(wu), None if bu is None else host64(bu)))
    assert err(H.cpu(), ref) <= BF16_TOL
    assert canaries_intact(buf, (M, I_))


# ---- split K: fewer large tiles than CUs, so K is shared between workgroups ----------------
# (the LDS-DMA kernel takes these once every CU gets at least 16 slices of 64, or 8 for plain
# products with K >= 2048). K ranges per tile: (1000, 16384, 1320) 8 (24 tiles), (2048, 8192, 1280) 6 (40 tiles),
# (4096, 8192, 1280) 3 (80 tiles), (1100, 3072, 2200) 5 (45 tiles), (1100, 4096, 1700) 7 (35
# tiles), (1400, 4096, 2500) 4 (60 tiles), (1024, 8192, 1280) 8 (20 tiles); ragged M and N.

@pytest.mark.parametrize("M,K,N", [(1000, 16384, 1320), (2048, 8192, 1280), (4096, 8192, 1280), (1100, 3072, 2200),
                                   (1100, 4096, 1700), (1400, 4096, 2500), (1024, 8192, 1280)])
def test_stream_k_linear(M, K, N):
    log_case("stream-K linear", M, K, N)
    x, w, b = I.activations(M, K, 321), I.weight(N, K, 322), I.bias(N, 323)
    buf, Y = canary_buffer((M, N), torch.bfloat16)
    tp.tp_linear_col(dev(x), dev(w), dev(b), Y, M, K, N, 1)
    torch.cuda.synchronize()
    rows = _sample_rows(M)
    ref = O.linear(host64(x)[rows], host64(w), host64(b))
    assert err(Y.cpu()[rows], ref) <= BF16_TOL
    assert canaries_intact(buf, (M, N))


def test_stream_k_partial_fp32():
    M, K, N = 1000, 16384, 1320
    log_case("stream-K fp32 partial", M, K, N)
    x, w = I.activations(M, K, 331), I.weight(N, K, 332)
    P = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tp.tp_linear_row_partial(dev(x), K, dev(w), P, M, K * 2, N, 2)
    torch.cuda.synchronize()
    rows = _sample_rows(M)
    ref = O.linear(host64(x)[rows], host64(w), None)
    assert err(P.cpu()[rows], ref) <= BF16_TOL


@pytest.mark.parametrize("M,K,I_", [(1000, 8192, 1000), (4096, 8192, 3584)])
def test_stream_k_swiglu(M, K, I_):
    log_case("stream-K swiglu", M, K, I_)
    x = I.activations(M, K, 341)
    wg, wu = I.weight(I_, K, 342), I.weight(I_, K, 343)
    bg, bu = I.bias(I_, 344), I.bias(I_, 345)
    buf, H = canary_buffer((M, I_), torch.bfloat16)
    tp.tp_mlp_shard(dev(x), dev(wg), dev(wu), dev(bg), dev(bu), None, H, None, M, K, I_, 1)
    torch.cuda.synchronize()
    rows = _sample_rows(M)
    xs = host64(x)[rows]
    ref = O.swiglu(O.linear(xs, host64(wg), host64(bg)), O.linear(xs, host64(wu), host64(bu)))
    assert err(H.cpu()[rows], ref) <= BF16_TOL
    assert canaries_intact(buf, (M, I_))
