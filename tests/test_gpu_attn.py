"""GPU parity of the head-local attention core (causal, grouped-query) against the fp64
oracle, through the C ABI: ragged token counts, both head sizes, the 70B shard's shape, and
the real chain QKV projection -> attention core -> O partial. From 4 query blocks of 128 on
(M >= 385) the causal core cuts its longer blocks into key ranges merged through the work
space (513, 700, 1000, 2048 tokens cover that path, the repeated 2048 call its counters), and
non-causal calls with few query blocks cut theirs too; where the ranges would need more than
one wave of resident workgroups, the work is cut into equal runs instead (2500 - 4096 tokens)."""
import numpy as np
import pytest
import torch

import oracle as O
import tensor_transformer_linear_col_amd as tp
import tp_inputs as I
from gpu_util import BF16_TOL, canaries_intact, canary_buffer, dev, err, host64, log_case

pytestmark = pytest.mark.gpu


def _core(qkv, M, hq, hk, d, causal):
    buf, A = canary_buffer((M, hq * d), torch.bfloat16)
    # tp_size = 1: the shard's own head counts
    tp.tp_attn_core_shard(dev(qkv), A, M, hq, hk, d, 1, causal)
    torch.cuda.synchronize()
    return buf, A


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("M", [1, 5, 32, 100, 128, 129, 300, 513, 1000])
def test_attention_core_matches_oracle(M, causal):
    hq, hk, d = 4, 2, 128
    log_case("attention core", M, hq, hk, d, causal)
    qkv = I.activations(M, (hq + 2 * hk) * d, 600 + M)
    buf, A = _core(qkv, M, hq, hk, d, causal)
    assert err(A, O.attention_core_shard(host64(qkv), hq, hk, d, causal)) <= BF16_TOL
    assert canaries_intact(buf, (M, hq * d))


@pytest.mark.parametrize("M", [7, 200, 700])
def test_attention_core_head_dim_64_one_kv_head(M):
    hq, hk, d = 8, 1, 64
    log_case("attention core d64", M, hq, hk, d)
    qkv = I.activations(M, (hq + 2 * hk) * d, 610 + M)
    buf, A = _core(qkv, M, hq, hk, d, True)
    assert err(A, O.attention_core_shard(host64(qkv), hq, hk, d, True)) <= BF16_TOL
    assert canaries_intact(buf, (M, hq * d))


def test_attention_core_70b_shard_shape_and_determinism():
    """8 query heads and 1 KV head of 128 (70B at TP = 8), 2048 tokens."""
    M, hq, hk, d = 2048, 8, 1, 128
    log_case("attention core 70b shard", M, hq, hk, d)
    qkv = I.activations(M, (hq + 2 * hk) * d, 620)
    _, A1 = _core(qkv, M, hq, hk, d, True)
    _, A2 = _core(qkv, M, hq, hk, d, True)
    assert torch.equal(A1, A2)
    assert err(A1, O.attention_core_shard(host64(qkv), hq, hk, d, True)) <= BF16_TOL


@pytest.mark.parametrize("M,hq,hk,d", [(2900, 8, 1, 128), (3000, 6, 2, 128), (2500, 16, 4, 64)])
def test_attention_core_equal_runs_schedule(M, hq, hk, d):
    """Causal prefill whose key ranges would need more than one wave of resident workgroups:
    the work order is cut into equal runs, so a workgroup takes pieces of two or more query
    blocks and a query block is merged from up to 4 runs (odd and even query-block counts,
    both head sizes). Every element against the oracle, a bitwise repeat (fixed merge order)."""
    log_case("attention core equal runs", M, hq, hk, d)
    qkv = I.activations(M, (hq + 2 * hk) * d, 630 + M)
    buf, A1 = _core(qkv, M, hq, hk, d, True)
    _, A2 = _core(qkv, M, hq, hk, d, True)
    assert torch.equal(A1, A2)
    assert err(A1, O.attention_core_shard(host64(qkv), hq, hk, d, True)) <= BF16_TOL
    assert canaries_intact(buf, (M, hq * d))


def test_attention_chain_qkv_core_o():
    """X -> QKV_r (column) -> attention core -> P_r (row) on every shard, summed + bo, against
    the unsharded chain with the real core."""
    nh, nkv, d, hid, p, M = 8, 2, 128, 512, 2, 96
    log_case("attention chain", M, nh, nkv, d, hid, p)
    shape = I.LayerShape("t", hidden=hid, n_heads=nh, n_kv_heads=nkv, head_dim=d, tp=p, seed=63)
    wt = I.attn_weights(shape)
    w64 = {k: host64(v) for k, v in wt.items()}
    x = I.activations(M, hid, 630)
    X = dev(x)
    hq, hk = nh // p, nkv // p
    parts = []
    for r in range(p):
        W_r = torch.empty((hq + 2 * hk) * d, hid, dtype=torch.bfloat16, device="cuda")
        b_r = torch.empty((hq + 2 * hk) * d, dtype=torch.bfloat16, device="cuda")
        tp.tp_shard_qkv(dev(wt["Wqkv"]), hid, nh, nkv, d, p, r, W_r)
        tp.tp_shard_qkv(dev(wt["bqkv"]), 1, nh, nkv, d, p, r, b_r)
        Wo_r = torch.empty(hid, hq * d, dtype=torch.bfloat16, device="cuda")
        tp.tp_shard_weight(dev(wt["Wo"]), hid, nh * d, p, r, 1, Wo_r)
        QKV_r = torch.empty(M, (hq + 2 * hk) * d, dtype=torch.bfloat16, device="cuda")
        A_r = torch.empty(M, hq * d, dtype=torch.bfloat16, device="cuda")
        P_r = torch.empty(M, hid, dtype=torch.bfloat16, device="cuda")
        tp.tp_attn_proj_shard(X, W_r, b_r, QKV_r, None, None, None, M, hid, nh, nkv, d, p)
        tp.tp_attn_core_shard(QKV_r, A_r, M, nh, nkv, d, p, True)
        tp.tp_attn_proj_shard(None, None, None, None, A_r, Wo_r, P_r, M, hid, nh, nkv, d, p)
        parts.append(P_r)
    Y = torch.empty(M, hid, dtype=torch.bfloat16, device="cuda")
    tp.tp_combine_sum(parts, dev(wt["bo"]), Y, M, hid)
    torch.cuda.synchronize()
    qkv = O.linear(host64(x), w64["Wqkv"], w64["bqkv"])
    a = O.attention_core_shard(qkv, nh, nkv, d, True)
    assert err(Y, O.linear(a, w64["Wo"], w64["bo"])) <= BF16_TOL


def _decode_sequence(S, nh, nkv, d, p, chunks, seed, capacity=None):
    """Feed a seeded S-token sequence of one shard's QKV rows through tp_attn_decode_shard in
    the given chunks; check every chunk's A_r against the rows of the oracle's causal pass over
    the whole sequence, and the caches against the sequence's K and V columns."""
    hq, hk = nh // p, tp.kv_heads_per_shard(nkv, p)
    qkv = I.activations(S, (hq + 2 * hk) * d, seed)
    full = O.attention_core_shard(host64(qkv), hq, hk, d, True)
    cap = capacity or S
    Kc = torch.zeros(cap, hk * d, dtype=torch.bfloat16, device="cuda")
    Vc = torch.zeros(cap, hk * d, dtype=torch.bfloat16, device="cuda")
    Q = dev(qkv)
    t = 0
    for m in chunks:
        log_case("attention decode", S, nh, nkv, d, p, t, m)
        buf, A = canary_buffer((m, hq * d), torch.bfloat16)
        tp.tp_attn_decode_shard(Q[t:t + m], Kc, Vc, t, A, m, nh, nkv, d, p)
        torch.cuda.synchronize()
        assert err(A, full[t:t + m]) <= BF16_TOL, (t, m)
        assert canaries_intact(buf, (m, hq * d))
        t += m
    assert torch.equal(Kc[:t].cpu(), qkv[:t, hq * d:(hq + hk) * d])
    assert torch.equal(Vc[:t].cpu(), qkv[:t, (hq + hk) * d:])


def test_attention_decode_70b_shard_over_cache():
    """70B at TP = 8 (8 query heads share 1 KV head of 128): a 300-token prompt through the
    cache, then single tokens and short chunks; the grouped heads are packed into one
    workgroup's rows."""
    _decode_sequence(400, 64, 8, 128, 8, [300, 1, 1, 7, 64, 27], 640, capacity=512)


def test_attention_decode_long_cache_cut_keys():
    """A 2000-token cache with 2 KV heads of 64: the keys are cut into ranges merged through the
    work space (one and sixteen new tokens)."""
    _decode_sequence(2033, 8, 4, 64, 2, [2000, 1, 16, 16], 650)


def test_attention_decode_prompt_equals_core():
    """An empty cache and the whole prompt in one call: the same attention as the core."""
    M, nh, nkv, d, p = 777, 32, 8, 128, 4
    hq, hk = nh // p, nkv // p
    qkv = I.activations(M, (hq + 2 * hk) * d, 660)
    Q = dev(qkv)
    A1 = torch.empty(M, hq * d, dtype=torch.bfloat16, device="cuda")
    A2 = torch.empty(M, hq * d, dtype=torch.bfloat16, device="cuda")
    Kc = torch.zeros(M, hk * d, dtype=torch.bfloat16, device="cuda")
    Vc = torch.zeros(M, hk * d, dtype=torch.bfloat16, device="cuda")
    log_case("attention decode prompt", M, nh, nkv, d, p)
    tp.tp_attn_core_shard(Q, A1, M, nh, nkv, d, p, True)
    tp.tp_attn_decode_shard(Q, Kc, Vc, 0, A2, M, nh, nkv, d, p)
    torch.cuda.synchronize()
    ref = O.attention_core_shard(host64(qkv), hq, hk, d, True)
    assert err(A1, ref) <= BF16_TOL
    assert err(A2, ref) <= BF16_TOL


_RNG_CASES = [  # (M, hq, hk, d, causal): seeded draws of token counts over the head layouts
    (m, hq, hk, d, causal)
    for (m, (hq, hk), d, causal) in zip(
        [3, 77, 191, 256, 385, 449, 640, 703],
        [(2, 1), (4, 2), (8, 1), (6, 3), (8, 2), (2, 2), (12, 4), (8, 1)],
        [64, 128, 128, 64, 128, 64, 128, 64],
        [True, False, True, True, False, True, True, False])
]


@pytest.mark.parametrize("M,hq,hk,d,causal", _RNG_CASES)
def test_attention_core_head_layouts(M, hq, hk, d, causal):
    log_case("attention core layout", M, hq, hk, d, causal)
    qkv = I.activations(M, (hq + 2 * hk) * d, 700 + M)
    buf, A = _core(qkv, M, hq, hk, d, causal)
    assert err(A, O.attention_core_shard(host64(qkv), hq, hk, d, causal)) <= BF16_TOL
    assert canaries_intact(buf, (M, hq * d))


@pytest.mark.parametrize("T,M,hq,hk,d", [(0, 5, 4, 4, 64), (17, 3, 6, 2, 128), (640, 200, 8, 1, 128),
                                         (1500, 40, 4, 2, 64)])
def test_attention_decode_shapes_and_determinism(T, M, hq, hk, d):
    """One step of M new tokens over a T-token cache: the oracle's rows, the appended cache rows,
    and a second identical call giving identical bits."""
    log_case("attention decode step", T, M, hq, hk, d)
    qkv = I.activations(T + M, (hq + 2 * hk) * d, 720 + T + M)
    Q = dev(qkv)
    full = O.attention_core_shard(host64(qkv), hq, hk, d, True)
    outs = []
    for _ in range(2):
        Kc = torch.zeros(T + M + 8, hk * d, dtype=torch.bfloat16, device="cuda")
        Vc = torch.zeros(T + M + 8, hk * d, dtype=torch.bfloat16, device="cuda")
        Kc[:T] = Q[:T, hq * d:(hq + hk) * d]
        Vc[:T] = Q[:T, (hq + hk) * d:]
        buf, A = canary_buffer((M, hq * d), torch.bfloat16)
        tp.tp_attn_decode_shard(Q[T:], Kc, Vc, T, A, M, hq, hk, d, 1)
        torch.cuda.synchronize()
        assert canaries_intact(buf, (M, hq * d))
        assert torch.equal(Kc[:T + M].cpu(), qkv[:, hq * d:(hq + hk) * d])
        assert torch.equal(Vc[:T + M].cpu(), qkv[:, (hq + hk) * d:])
        assert not Kc[T + M:].any().item()  # nothing past the new rows
        outs.append(A.clone())
    assert err(outs[0], full[T:]) <= BF16_TOL
    assert torch.equal(outs[0], outs[1])


def test_attention_core_70b_shard_full_size():
    """The size bench.py times: 8 query heads and 1 KV head of 128 over 4096 tokens, causal, in
    its launch configuration (query blocks cut into up to 3 key ranges, largest first), against
    the oracle on every element."""
    M, nh, nkv, d, p = 4096, 64, 8, 128, 8
    hq, hk = nh // p, nkv // p
    log_case("attention core full size", M, hq, hk, d)
    qkv = I.activations(M, (hq + 2 * hk) * d, 680)
    Q = dev(qkv)
    buf, A = canary_buffer((M, hq * d), torch.bfloat16)
    tp.tp_attn_core_shard(Q, A, M, nh, nkv, d, p, True)
    torch.cuda.synchronize()
    assert err(A, O.attention_core_shard(host64(qkv), hq, hk, d, True)) <= BF16_TOL
    assert canaries_intact(buf, (M, hq * d))


@pytest.mark.parametrize("T,M", [(4096, 1), (32768, 16)])
def test_attention_decode_bench_sizes(T, M):
    """The decode steps bench.py times (70B TP=8 shard: 8 query heads over 1 KV head of 128):
    M new tokens over a T-token cache, against the oracle's decode step."""
    nh, nkv, d, p = 64, 8, 128, 8
    hq, hk = nh // p, nkv // p
    log_case("attention decode bench size", T, M)
    cache = I.activations(T, 2 * hk * d, 690 + M)
    new = I.activations(M, (hq + 2 * hk) * d, 691 + M)
    Kc = torch.zeros(T + M, hk * d, dtype=torch.bfloat16, device="cuda")
    Vc = torch.zeros(T + M, hk * d, dtype=torch.bfloat16, device="cuda")
    Kc[:T] = dev(cache[:, :hk * d])
    Vc[:T] = dev(cache[:, hk * d:])
    buf, A = canary_buffer((M, hq * d), torch.bfloat16)
    tp.tp_attn_decode_shard(dev(new), Kc, Vc, T, A, M, nh, nkv, d, p)
    torch.cuda.synchronize()
    c64 = host64(cache)
    ref, _, _ = O.attention_decode_shard(host64(new), c64[:, :hk * d], c64[:, hk * d:], hq, hk, d)
    assert err(A, ref) <= BF16_TOL
    assert canaries_intact(buf, (M, hq * d))
