"""GPU parity of the pages' GELU FFN shard (column layer, erf GELU, row layer) against
the fp64 oracle, through the C ABI: decode-sized and prefill-sized token counts, bf16
and fp32, each shard and the combined result."""
import numpy as np
import pytest
import torch

import oracle as O
import tensor_transformer_linear_col_amd as tp
import tp_inputs as I
from gpu_util import BF16_TOL, F32_TOL, canaries_intact, canary_buffer, dev, err, host64, log_case

pytestmark = pytest.mark.gpu


def _run_shards(x, wt, M, h, inter, p, dtype=torch.bfloat16, with_p=True):
    i = inter // p
    X = dev(x)
    out = []
    for r in range(p):
        sl = slice(r * i, (r + 1) * i)
        W1 = dev(wt["W1"][sl])
        b1 = dev(wt["b1"][sl]) if "b1" in wt else None
        W2 = dev(wt["W2"][:, sl])
        buf, H = canary_buffer((M, i), dtype)
        P = torch.empty(M, h, dtype=dtype, device="cuda") if with_p else None
        tp.tp_ffn_gelu_shard(X, W1, b1, W2 if with_p else None, H, P, M, h, inter, p)
        out.append((buf, H, P))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("M", [1, 4, 17, 40, 64, 65, 300])
def test_gelu_ffn_shards_bf16(M):
    h, inter, p = 512, 1536, 2
    log_case("gelu ffn bf16", M, h, inter, p)
    shape = I.LayerShape("t", hidden=h, intermediate=inter, tp=p, seed=40)
    wt = I.gelu_ffn_weights(shape)
    x = I.activations(M, h, 400 + M)
    w64 = {k: host64(v) for k, v in wt.items()}
    ref_shards = O.ffn_gelu_shards(host64(x), w64["W1"], w64["W2"], p, w64["b1"])
    outs = _run_shards(x, wt, M, h, inter, p)
    for r, ((buf, H, P), (h_ref, p_ref)) in enumerate(zip(outs, ref_shards)):
        assert err(H, h_ref) <= BF16_TOL
        assert canaries_intact(buf, (M, inter // p))
        # the row layer is checked on the H the GPU actually produced
        assert err(P, O.row_partial(host64(H), O.row_shard(w64["W2"], p, r))) <= BF16_TOL
    Y = torch.empty(M, h, dtype=torch.bfloat16, device="cuda")
    tp.tp_combine_sum([P for _, _, P in outs], dev(wt["b2"]), Y, M, h)
    torch.cuda.synchronize()
    assert err(Y, O.ffn_gelu(host64(x), w64["W1"], w64["W2"], w64["b1"], w64["b2"])) <= BF16_TOL


def test_gelu_ffn_fp32():
    M, h, inter, p = 5, 64, 96, 2
    log_case("gelu ffn fp32", M, h, inter, p)
    shape = I.LayerShape("t", hidden=h, intermediate=inter, tp=p, seed=41)
    wt = I.gelu_ffn_weights(shape, dtype=torch.float32)
    x = I.activations(M, h, 411, dtype=torch.float32)
    outs = _run_shards(x, wt, M, h, inter, p, dtype=torch.float32)
    Y = torch.empty(M, h, dtype=torch.float32, device="cuda")
    tp.tp_combine_sum([P for _, _, P in outs], dev(wt["b2"]), Y, M, h)
    torch.cuda.synchronize()
    w64 = {k: host64(v) for k, v in wt.items()}
    assert err(Y, O.ffn_gelu(host64(x), w64["W1"], w64["W2"], w64["b1"], w64["b2"])) <= F32_TOL


def test_gelu_ffn_pages_shape_batch4_tp2():
    """The listing's example: 4096 -> 11008 -> 4096 at batch 4, here at TP = 2."""
    s = I.PAGES_FFN_GELU_TP2
    M = s.tokens[0]
    log_case("gelu ffn pages shape", M, s.hidden, s.intermediate, s.tp)
    wt = I.gelu_ffn_weights(s)
    x = I.activations(M, s.hidden, I.activation_seed(s.seed, M))
    outs = _run_shards(x, wt, M, s.hidden, s.intermediate, s.tp)
    Y = torch.empty(M, s.hidden, dtype=torch.bfloat16, device="cuda")
    tp.tp_combine_sum([P for _, _, P in outs], dev(wt["b2"]), Y, M, s.hidden)
    torch.cuda.synchronize()
    assert tuple(Y.shape) == (4, 4096)   # the listing prints the output shape
    w64 = {k: host64(v) for k, v in wt.items()}
    assert err(Y, O.ffn_gelu(host64(x), w64["W1"], w64["W2"], w64["b1"], w64["b2"])) <= BF16_TOL


def test_gelu_ffn_prefill_sampled_rows():
    """2048 tokens: the large-tile MFMA kernels, checked on sampled token rows."""
    s = I.PAGES_FFN_GELU_TP2
    M, h, inter, p = 2048, s.hidden, s.intermediate, s.tp
    log_case("gelu ffn prefill", M, h, inter, p)
    wt = I.gelu_ffn_weights(s)
    x = I.activations(M, h, I.activation_seed(s.seed, M))
    outs = _run_shards(x, wt, M, h, inter, p)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(5).choice(M, 6, replace=False)]))
    w64 = {k: host64(v) for k, v in wt.items()}
    xs = host64(x)[rows]
    for r, (buf, H, P) in enumerate(outs):
        w1_r, b1_r = O.col_shard(w64["W1"], w64["b1"], p, r)
        assert err(H.cpu()[rows], O.gelu(O.linear(xs, w1_r, b1_r))) <= BF16_TOL
        assert canaries_intact(buf, (M, inter // p))
        assert err(P.cpu()[rows], O.row_partial(host64(H.cpu()[rows]), O.row_shard(w64["W2"], p, r))) <= BF16_TOL
