"""GPU parity of the few-token GEMV path (1-4 tokens with fewer 16-feature row groups than
CUs, e.g. the 70B QKV shard at TP = 8): every output element against the fp64 oracle,
across ragged K (each wave's K range ends mid-chunk), every epilogue, fp32 partials,
strided token rows, one to 4095 features, with canaries after the output and a bitwise
repeat."""
import numpy as np
import pytest
import torch

import oracle as O
import tensor_transformer_linear_col_amd as tp
import tp_inputs as I
from gpu_util import BF16_TOL, canaries_intact, canary_buffer, dev, err, host64, log_case

pytestmark = pytest.mark.gpu

BF = torch.bfloat16

# (K, N): K tails inside a wave's range (1000, 5504 + 8), one chunk per wave (4096), two (8192),
# four (16384), tiny K (8, 64); N from a single feature to just under 16 x 256.
SHAPES = [(8, 1), (64, 17), (1000, 255), (4096, 256), (4096, 1280), (5512, 1000), (8192, 1280),
          (16384, 300), (2048, 4095)]


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("K,N", SHAPES)
def test_gemv_linear(K, N, M):
    log_case("gemv linear", M, K, N)
    x, w, b = I.activations(M, K, 700 + M), I.weight(N, K, 701), I.bias(N, 702)
    buf, Y = canary_buffer((M, N), BF)
    tp.tp_linear_col(dev(x), dev(w), dev(b), Y, M, K, N, 1)
    Y2 = torch.empty(M, N, dtype=BF, device="cuda")
    tp.tp_linear_col(dev(x), dev(w), dev(b), Y2, M, K, N, 1)
    torch.cuda.synchronize()
    assert err(Y.cpu(), O.linear(host64(x), host64(w), host64(b))) <= BF16_TOL
    assert canaries_intact(buf, (M, N))
    assert torch.equal(Y, Y2)


@pytest.mark.parametrize("M", [1, 3, 4])
@pytest.mark.parametrize("K,I_", [(4096, 1000), (8192, 1536), (1000, 77)])
@pytest.mark.parametrize("bias", [False, True])
def test_gemv_swiglu(K, I_, M, bias):
    log_case("gemv swiglu", M, K, I_, bias)
    x = I.activations(M, K, 710 + M)
    wg, wu = I.weight(I_, K, 711), I.weight(I_, K, 712)
    bg, bu = (I.bias(I_, 713), I.bias(I_, 714)) if bias else (None, None)
    buf, H = canary_buffer((M, I_), BF)
    tp.tp_mlp_shard(dev(x), dev(wg), dev(wu), dev(bg), dev(bu), None, H, None, M, K, I_, 1)
    torch.cuda.synchronize()
    xs = host64(x)
    ref = O.swiglu(O.linear(xs, host64(wg), None if bg is None else host64(bg)),
                   O.linear(xs, host64(wu), None if bu is None else host64(bu)))
    assert err(H.cpu(), ref) <= BF16_TOL
    assert canaries_intact(buf, (M, I_))


@pytest.mark.parametrize("M", [1, 4])
def test_gemv_gelu_and_fp32_partial(M):
    K, N = 4096, 1200
    log_case("gemv gelu + fp32 partial", M, K, N)
    x, w, b = I.activations(M, K, 720 + M), I.weight(N, K, 721), I.bias(N, 722)
    H = torch.empty(M, N, dtype=BF, device="cuda")
    tp.tp_ffn_gelu_shard(dev(x), dev(w), dev(b), None, H, None, M, K, N, 1)
    torch.cuda.synchronize()
    assert err(H.cpu(), O.gelu(O.linear(host64(x), host64(w), host64(b)))) <= BF16_TOL
    # a row partial with fp32 output, X read through a row stride (the rank's slice of a full X)
    xf = I.activations(M, 2 * K, 723)
    P = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tp.tp_linear_row_partial(dev(xf)[:, K:], 2 * K, dev(w), P, M, 2 * K, N, 2)
    torch.cuda.synchronize()
    assert err(P.cpu(), O.linear(host64(xf)[:, K:], host64(w))) <= BF16_TOL


def test_gemv_matches_the_qkv_shard_oracle_per_shard():
    """The 70B attention projection at TP = 8, one token: each shard's QKV against the oracle's
    head-split shard, every element."""
    shape = I.LLAMA70B_ATTN_TP8
    h, nh, nkv, d, p = shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.tp
    log_case("gemv qkv shards", 1)
    wt = I.attn_weights(shape, with_bias=True)
    x = I.activations(1, h, 730)
    Wqkv, bqkv, X = dev(wt["Wqkv"]), dev(wt["bqkv"]), dev(x)
    nq = (nh // p + 2 * nkv // p) * d
    for r in range(p):
        W_r = torch.empty(nq, h, dtype=BF, device="cuda")
        b_r = torch.empty(nq, dtype=BF, device="cuda")
        tp.tp_shard_qkv(Wqkv, h, nh, nkv, d, p, r, W_r)
        tp.tp_shard_qkv(bqkv, 1, nh, nkv, d, p, r, b_r)
        Q = torch.empty(1, nq, dtype=BF, device="cuda")
        tp.tp_attn_proj_shard(X, W_r, b_r, Q, None, None, None, 1, h, nh, nkv, d, p)
        torch.cuda.synchronize()
        w_ref, b_ref = O.qkv_shard(host64(wt["Wqkv"]), host64(wt["bqkv"]), nh, nkv, d, p, r)
        assert err(Q.cpu(), O.col_linear(host64(x), w_ref, b_ref)) <= BF16_TOL
