"""Seeded sweep across the kernel-selection boundaries of the linear products: 1-4 tokens with
few or many row groups (GEMV or MFMA decode kernel), 5-64 tokens (MFMA decode tiles), 65-300
tokens (register-staged prefill tiles) and large prefill shapes (LDS-DMA tiles, split-K), each
product kind (plain column, column + bias, SwiGLU pair with and without biases, GELU, row
partial in bf16 and fp32), compared on every element with the fp64 oracle. The shapes are
drawn once from a fixed seed."""
import numpy as np
import pytest
import torch

import oracle as O
import tensor_transformer_linear_col_amd as tp
import tp_inputs as I
from gpu_util import BF16_TOL, canaries_intact, canary_buffer, dev, err, host64, log_case

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _cases():
    rng = np.random.default_rng(2024)
    kinds = ["col", "col_bias", "swiglu", "swiglu_bias", "gelu", "row_bf16", "row_f32"]
    out = []
    for M in (1, 2, 3, 4, 5, 8, 13, 16, 17, 33, 48, 64, 65, 130, 300):
        for _ in range(2):
            kind = kinds[rng.integers(len(kinds))]
            K = int(rng.integers(1, 1024)) * 8
            N = int(rng.integers(1, 5000))
            out.append((M, K, N, kind))
    # large prefill shapes on the LDS-DMA kernel: whole waves of tiles, and split-K remainders;
    # then long K on few tiles (8 K ranges of 10 or 8 tiles), the SwiGLU pair without biases in
    # 4 ranges, and short K kept on register-staged tiles
    out += [(512, 4096, 16384, "col"), (1024, 8192, 1536, "col_bias"), (700, 6144, 2000, "swiglu_bias"),
            (2048, 2048, 4100, "row_f32"), (512, 8192, 1280, "col"), (300, 4096, 1000, "row_f32"),
            (512, 8192, 3584, "swiglu"), (1024, 1024, 8192, "col")]
    return out


CASES = _cases()


@pytest.mark.parametrize("M,K,N,kind", CASES, ids=[f"{c[3]}-M{c[0]}-K{c[1]}-N{c[2]}" for c in CASES])
def test_routing_sweep(M, K, N, kind):
    log_case("routing sweep", M, K, N, kind)
    seed = 9000 + M * 7 + K + N
    x = I.activations(M, K, seed)
    w = I.weight(N, K, seed + 1)
    xs, w64 = host64(x), host64(w)
    if kind in ("col", "col_bias", "gelu"):
        b = I.bias(N, seed + 2) if kind != "col" else None
        buf, Y = canary_buffer((M, N), BF)
        if kind == "gelu":
            tp.tp_ffn_gelu_shard(dev(x), dev(w), dev(b), None, Y, None, M, K, N, 1)
            ref = O.gelu(O.linear(xs, w64, host64(b)))
        else:
            tp.tp_linear_col(dev(x), dev(w), dev(b), Y, M, K, N, 1)
            ref = O.linear(xs, w64, None if b is None else host64(b))
    elif kind in ("swiglu", "swiglu_bias"):
        wu = I.weight(N, K, seed + 3)
        bg, bu = (I.bias(N, seed + 4), I.bias(N, seed + 5)) if kind == "swiglu_bias" else (None, None)
        buf, Y = canary_buffer((M, N), BF)
        tp.tp_mlp_shard(dev(x), dev(w), dev(wu), dev(bg), dev(bu), None, Y, None, M, K, N, 1)
        ref = O.swiglu(O.linear(xs, w64, None if bg is None else host64(bg)),
                       O.linear(xs, host64(wu), None if bu is None else host64(bu)))
    else:
        dt = BF if kind == "row_bf16" else torch.float32
        buf, Y = canary_buffer((M, N), dt)
        tp.tp_linear_row_partial(dev(x), K, dev(w), Y, M, K, N, 1)
        ref = O.linear(xs, w64)
    torch.cuda.synchronize()
    assert err(Y.cpu(), ref) <= BF16_TOL
    assert canaries_intact(buf, (M, N))
