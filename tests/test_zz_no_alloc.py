"""The allocation-free MLP entry point (tp_mlp_shard_noalloc), through the C ABI: its split
reductions take their partials and counters from the library's fixed per-GPU scratch array.
It must match tp_mlp_shard (same kernels, same reduction order: bit-identical) on two calls
in a row, the second with a smaller input, and refuse a call whose split needs more scratch
than the array holds without enqueuing anything."""
import pytest
import torch

import oracle as O
import tensor_transformer_linear_col_amd as tp
import tp_inputs as I
from gpu_util import BF16_TOL, dev, err, host64, log_case

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _shard(M, hidden, inter, p, r, seed, bias=True):
    shape = I.LayerShape("noalloc", hidden=hidden, intermediate=inter, tp=p, seed=seed)
    wt = I.ffn_weights(shape, with_bias=bias)
    i = inter // p
    sl = slice(r * i, (r + 1) * i)
    w = {"Wg": wt["Wg"][sl], "Wu": wt["Wu"][sl], "Wd": wt["Wd"][:, sl],
         "bg": wt["bg"][sl] if bias else None, "bu": wt["bu"][sl] if bias else None}
    x = I.activations(M, hidden, seed * 1000 + M)
    return x, w, i


def _run(fn, X, w, M, hidden, inter, p, i):
    H = torch.full((M, i), float("nan"), dtype=BF, device="cuda")
    P = torch.full((M, hidden), float("nan"), dtype=BF, device="cuda")
    fn(X, w["Wg"], w["Wu"], w["bg"], w["bu"], w["Wd"], H, P, M, hidden, inter, p)
    return H, P


# (M, hidden, intermediate, tp), each call smaller than the one before: the 7B FFN shard at 64
# tokens (both products on LDS-staged tiles whose K ranges meet in fp32 partials), at 8 tokens
# (its down product cuts K across workgroups), then a smaller shard at 6 tokens (its gate/up
# product cuts K).
CALLS = [(64, 4096, 11008, 2), (8, 4096, 11008, 2), (6, 1024, 2816, 4)]


def test_noalloc_matches_the_reserved_entry_point_on_two_calls():
    for n, (M, hidden, inter, p) in enumerate(CALLS):
        log_case("noalloc call", n, M, hidden, inter, p)
        x, w, i = _shard(M, hidden, inter, p, p - 1, seed=60 + n)
        X, wd = dev(x), {k: dev(v) for k, v in w.items()}
        with tp.tp_plan() as need:
            tp.tp_mlp_shard(X, wd["Wg"], wd["Wu"], wd["bg"], wd["bu"], wd["Wd"],
                            torch.empty(M, i, dtype=BF, device="cuda"), torch.empty(M, hidden, dtype=BF, device="cuda"),
                            M, hidden, inter, p)
        assert need.partial_bytes > 0  # a split reduction runs
        H0, P0 = _run(tp.tp_mlp_shard, X, wd, M, hidden, inter, p, i)
        H1, P1 = _run(tp.tp_mlp_shard_noalloc, X, wd, M, hidden, inter, p, i)
        torch.cuda.synchronize()
        assert torch.equal(H1, H0) and torch.equal(P1, P0)
        xs, w64 = host64(x), {k: host64(v) for k, v in w.items()}
        h_ref = O.swiglu(O.linear(xs, w64["Wg"], w64["bg"]), O.linear(xs, w64["Wu"], w64["bu"]))
        assert err(H1.cpu(), h_ref) <= BF16_TOL
        assert err(P1.cpu(), O.linear(host64(H1.cpu()), w64["Wd"])) <= BF16_TOL


def test_noalloc_refuses_a_split_larger_than_its_scratch():
    """2048 tokens, hidden 8192, 512 intermediate features per shard: the gate/up product runs
    split-K over 32 tiles x 4 K ranges = 32 MiB of fp32 partials, more than the 16 MiB array."""
    M, hidden, inter, p = 2048, 8192, 4096, 8
    log_case("noalloc refusal", M, hidden, inter, p)
    x, w, i = _shard(M, hidden, inter, p, 0, seed=70, bias=False)
    X, wd = dev(x), {k: dev(v) for k, v in w.items()}
    with pytest.raises(tp.TPError) as e:
        _run(tp.tp_mlp_shard_noalloc, X, wd, M, hidden, inter, p, i)
    assert e.value.status == tp.TP_ERR_WORKSPACE
    H = torch.full((M, i), float("nan"), dtype=BF, device="cuda")
    with pytest.raises(tp.TPError):
        tp.tp_mlp_shard_noalloc(X, wd["Wg"], wd["Wu"], None, None, None, H, None, M, hidden, inter, p)
    torch.cuda.synchronize()
    assert torch.isnan(H).all()
