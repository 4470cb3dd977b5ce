"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's own formula: they compare it with
values printed on the pages, with explicit-loop brute force (math.fsum), with
closed forms and special cases, and with the invariants the pages state.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import tp_inputs as I
from conftest import read_golden


def _toy():
    x, w, b = I.toy_layer()
    return I.as_numpy_f64(x), I.as_numpy_f64(w), I.as_numpy_f64(b)


# --- "Tensor parallel serving", "Simulating the split ...", block "Output" ----------

def test_toy_full_output_matches_printed_values():
    g = read_golden("toy_tp2.txt")
    x, w, b = _toy()
    full = O.linear(x, w, b)
    printed = np.array([float(v) for v in g["full_output_round4"]])
    assert full.shape == (1, 6)
    np.testing.assert_array_equal(np.round(full[0], 4), printed)


def test_toy_column_split_concat_matches_printed_values_and_is_exact():
    g = read_golden("toy_tp2.txt")
    x, w, b = _toy()
    parts = []
    for r in range(2):
        w_r, b_r = O.col_shard(w, b, 2, r)
        parts.append(O.col_linear(x, w_r, b_r))
    combined = O.concat(parts)
    printed = np.array([float(v) for v in g["combined_output_round4"]])
    np.testing.assert_array_equal(np.round(combined[0], 4), printed)
    # "outputs match exactly: True": each element is the same dot product in the same order.
    assert g["outputs_match"] == ["True"]
    np.testing.assert_array_equal(combined, O.linear(x, w, b))


def test_toy_shard_sizes_24_of_48():
    g = read_golden("toy_tp2.txt")
    _, w, b = _toy()
    for r, key in enumerate(("gpu0_held", "gpu1_held")):
        w_r, _ = O.col_shard(w, b, 2, r)
        held, total = (int(v) for v in g[key])
        assert w_r.size == held and w.size == total


def test_toy_row_split_sum_plus_bias_equals_unsharded():
    """Row parallelism: partial sums over input slices, summed, bias once ("Common mistakes")."""
    g = read_golden("toy_tp2.txt")
    x, w, b = _toy()
    parts = []
    for r in range(2):
        parts.append(O.row_partial(O.input_slice(x, 2, r), O.row_shard(w, 2, r)))
        assert O.row_shard(w, 2, r).shape == (6, 4)
    y = O.combine_sum(parts, b)
    full = O.linear_fsum(x, w, b)
    assert O.rel_err(y, full) <= 1e-12
    printed = np.array([float(v) for v in g["full_output_round4"]])
    np.testing.assert_array_equal(np.round(y[0], 4), printed)


def test_toy_row_partials_by_bruteforce():
    x, w, _ = _toy()
    for r in range(2):
        xs, ws = O.input_slice(x, 2, r), O.row_shard(w, 2, r)
        np.testing.assert_allclose(O.row_partial(xs, ws), O.linear_fsum(xs, ws), rtol=0, atol=1e-14)


# --- brute force on tiny inputs ------------------------------------------------------

@pytest.mark.parametrize("m,k,n", [(1, 1, 1), (1, 8, 6), (3, 5, 7), (4, 16, 9), (5, 33, 2)])
def test_linear_matches_fsum_bruteforce(m, k, n):
    g = torch.Generator().manual_seed(1000 + m * 100 + k * 10 + n)
    x = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = torch.randn(n, k, generator=g).to(torch.bfloat16)
    b = torch.randn(n, generator=g).to(torch.bfloat16)
    xf, wf, bf = (I.as_numpy_f64(t) for t in (x, w, b))
    np.testing.assert_allclose(O.linear(xf, wf, bf), O.linear_fsum(xf, wf, bf), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(O.linear(xf, wf), O.linear_fsum(xf, wf), rtol=1e-13, atol=1e-13)


def test_linear_entry_spot_matches():
    x = I.as_numpy_f64(I.activations(3, 40, seed=11))
    w = I.as_numpy_f64(I.weight(5, 40, seed=12))
    b = I.as_numpy_f64(I.bias(5, seed=13))
    y = O.linear(x, w, b)
    for m in range(3):
        for n in range(5):
            assert abs(O.linear_entry(x[m], w[n], b[n]) - y[m, n]) <= 1e-14


# --- closed-form special cases ---------------------------------------------------------

def test_identity_weight_returns_input_plus_bias():
    x = I.as_numpy_f64(I.activations(4, 16, seed=21))
    b = I.as_numpy_f64(I.bias(16, seed=22))
    np.testing.assert_array_equal(O.linear(x, np.eye(16)), x)
    np.testing.assert_array_equal(O.linear(x, np.eye(16), b), x + b)


def test_one_hot_input_selects_weight_column():
    w = I.as_numpy_f64(I.weight(7, 12, seed=23))
    b = I.as_numpy_f64(I.bias(7, seed=24))
    for k in range(12):
        e = np.zeros((1, 12))
        e[0, k] = 1.0
        np.testing.assert_array_equal(O.linear(e, w, b)[0], w[:, k] + b)


def test_non_square_orientation():
    """Y has out_features columns: a transposed operand cannot even produce this shape."""
    x = np.ones((2, 3))
    w = np.array([[1.0, 2.0, 3.0]])  # [out=1, in=3]
    np.testing.assert_array_equal(O.linear(x, w), [[6.0], [6.0]])


def test_silu_closed_forms():
    # sigmoid(ln 3) = 3/4, so silu(ln 3) = (3/4) ln 3 and silu(-ln 3) = -(1/4) ln 3.
    ln3 = math.log(3.0)
    z = np.array([0.0, ln3, -ln3, 40.0, -40.0])
    s = O.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 0.75 * ln3) < 1e-15
    assert abs(s[2] + 0.25 * ln3) < 1e-15
    assert abs(s[3] - 40.0) < 1e-12            # silu(z) -> z for z >> 0
    assert abs(s[4]) < 1e-15                   # silu(z) -> 0 for z << 0
    zz = np.linspace(-6, 6, 97)
    np.testing.assert_allclose(O.silu(zz) - O.silu(-zz), zz, atol=1e-14)  # z*s(z) + z*s(-z) = z


def test_swiglu_special_cases():
    u = np.array([[1.5, -2.0, 3.0]])
    np.testing.assert_array_equal(O.swiglu(np.zeros((1, 3)), u), np.zeros((1, 3)))
    np.testing.assert_allclose(O.swiglu(np.full((1, 3), 50.0), u), 50.0 * u, rtol=1e-15)
    ln3 = math.log(3.0)
    np.testing.assert_allclose(O.swiglu(np.full((1, 3), ln3), u), 0.75 * ln3 * u, rtol=1e-15)


def test_gelu_closed_forms():
    # gelu(z) = z * Phi(z); tabulated standard normal CDF: Phi(1) = 0.8413447460685429,
    # Phi(2) = 0.9772498680518208, Phi(-1) = 1 - Phi(1).
    z = np.array([0.0, 1.0, -1.0, 2.0, 10.0, -10.0])
    g = O.gelu(z)
    assert g[0] == 0.0
    assert abs(g[1] - 0.8413447460685429) < 1e-15
    assert abs(g[2] + (1.0 - 0.8413447460685429)) < 1e-15
    assert abs(g[3] - 2.0 * 0.9772498680518208) < 1e-15
    assert abs(g[4] - 10.0) < 1e-12             # gelu(z) -> z for z >> 0
    assert abs(g[5]) < 1e-20                    # gelu(z) -> 0 for z << 0
    zz = np.linspace(-6, 6, 97)
    np.testing.assert_allclose(O.gelu(zz) - O.gelu(-zz), zz, atol=1e-14)  # z*Phi(z) + z*Phi(-z) = z


# --- invariants the pages state ---------------------------------------------------------

def test_bias_added_to_every_partial_is_off_by_p_minus_1_times_b():
    """Bias once, after the sum (the listing's RowParallelLinear adds it after all_reduce)."""
    p = 4
    x = I.as_numpy_f64(I.activations(3, 32, seed=31))
    w = I.as_numpy_f64(I.weight(10, 32, seed=32))
    b = I.as_numpy_f64(I.bias(10, seed=33))
    parts = [O.row_partial(O.input_slice(x, p, r), O.row_shard(w, p, r)) for r in range(p)]
    right = O.combine_sum(parts, b)
    wrong = O.combine_sum([pr + b[None, :] for pr in parts])
    np.testing.assert_allclose(wrong - right, np.broadcast_to((p - 1) * b, right.shape), atol=1e-13)
    np.testing.assert_allclose(right, O.linear_fsum(x, w, b), atol=1e-13)


def test_wrong_combine_gives_confidently_wrong_numbers():
    """Row split combined by concat (or column split by sum) is wrong, not an error."""
    p = 2
    x = I.as_numpy_f64(I.activations(2, 8, seed=41))
    w = I.as_numpy_f64(I.weight(6, 8, seed=42))
    ref = O.linear(x, w)
    row_parts = [O.row_partial(O.input_slice(x, p, r), O.row_shard(w, p, r)) for r in range(p)]
    assert O.concat(row_parts).shape != ref.shape or not np.allclose(O.concat(row_parts), ref)
    col_parts = [O.col_linear(x, O.col_shard(w, None, p, r)[0]) for r in range(p)]
    assert not np.allclose(O.combine_sum(col_parts), ref[:, :3])


def test_uneven_split_9_equals_5_plus_4():
    """'Try it yourself': OUT_FEATURES = 9 split 5 + 4 still matches exactly."""
    x, w, b = (I.as_numpy_f64(t) for t in I.toy_layer_uneven(9))
    parts = [O.col_linear(x, w_r, b_r) for w_r, b_r in O.col_shard_uneven(w, b, (5, 4))]
    np.testing.assert_array_equal(O.concat(parts), O.linear(x, w, b))


def test_uneven_row_split_sum_equals_unsharded():
    """The row layer split unevenly (5 + 3 + 8 inputs): the partials still sum to X W^T."""
    x = I.as_numpy_f64(I.activations(3, 16, seed=51))
    w = I.as_numpy_f64(I.weight(7, 16, seed=52))
    widths = (5, 3, 8)
    parts = [O.row_partial(x_r, w_r) for x_r, w_r in zip(O.input_slices_uneven(x, widths), O.row_shard_uneven(w, widths))]
    np.testing.assert_allclose(O.combine_sum(parts), O.linear(x, w), rtol=1e-13, atol=1e-15)
    # brute force on every entry
    ref = O.linear_fsum(x, w)
    np.testing.assert_allclose(O.combine_sum(parts), ref, rtol=1e-13, atol=1e-15)
    with pytest.raises(ValueError):
        O.row_shard_uneven(w, (5, 3, 7))
    with pytest.raises(ValueError):
        O.blocks_of(16, (16, 0))


def test_kv_heads_replicated_when_more_shards_than_kv_heads():
    """A reading (the pages only require TP to divide the heads): with p a multiple of the
    KV head count, KV head h lives on the p/G consecutive shards h*p/G .. (h+1)*p/G - 1."""
    assert [O.kv_heads_of(8, 16, r) for r in range(16)] == [[r // 2] for r in range(16)]
    assert [O.kv_heads_of(8, 4, r) for r in range(4)] == [[2 * r, 2 * r + 1] for r in range(4)]
    assert O.kv_heads_of(2, 8, 7) == [1]
    with pytest.raises(ValueError):
        O.kv_heads_of(8, 12, 0)
    nh, nkv, d, hid, p = 8, 2, 4, 16, 4
    shape = I.LayerShape("t", hidden=hid, n_heads=nh, n_kv_heads=nkv, head_dim=d, tp=p, seed=12)
    wt = {k: I.as_numpy_f64(v) for k, v in I.attn_weights(shape).items()}
    x = I.as_numpy_f64(I.activations(3, hid, seed=121))
    full = O.linear(x, wt["Wqkv"], wt["bqkv"])
    hq = nh // p
    for r in range(p):
        w_r, b_r = O.qkv_shard(wt["Wqkv"], wt["bqkv"], nh, nkv, d, p, r)
        assert w_r.shape == ((hq + 2) * d, hid)
        y = O.col_linear(x, w_r, b_r)
        h = r * nkv // p
        np.testing.assert_array_equal(y[:, :hq * d], full[:, r * hq * d:(r + 1) * hq * d])
        np.testing.assert_array_equal(y[:, hq * d:(hq + 1) * d], full[:, (nh + h) * d:(nh + h + 1) * d])
        np.testing.assert_array_equal(y[:, (hq + 1) * d:], full[:, (nh + nkv + h) * d:(nh + nkv + h + 1) * d])


def test_qkv_segments_and_concat_with_replicated_kv_heads():
    """Replication (a reading, parity unpinned by the pages): with p a multiple of G each shard's
    K and V segments are one head wide; every replica's K/V segment equals that KV head's
    columns of the unsharded QKV, and the segment concat with each head taken from its first
    holder is the unsharded QKV. The sharded layer chain then matches the unsharded one."""
    assert O.qkv_segments(64, 8, 128, 16) == (512, 128, 128)
    assert O.qkv_segments(64, 8, 128, 8) == (1024, 128, 128)
    assert O.qkv_segments(64, 8, 128, 4) == (2048, 256, 256)
    assert O.qkv_segments(16, 2, 64, 8) == (128, 64, 64)
    with pytest.raises(ValueError):
        O.qkv_segments(64, 8, 128, 12)
    nh, nkv, d, hid, p = 8, 2, 4, 16, 8
    shape = I.LayerShape("t", hidden=hid, n_heads=nh, n_kv_heads=nkv, head_dim=d, tp=p, seed=13)
    wt = {k: I.as_numpy_f64(v) for k, v in I.attn_weights(shape).items()}
    x = I.as_numpy_f64(I.activations(3, hid, seed=131))
    full = O.linear(x, wt["Wqkv"], wt["bqkv"])
    seg = O.qkv_segments(nh, nkv, d, p)
    parts = [O.col_linear(x, *O.qkv_shard(wt["Wqkv"], wt["bqkv"], nh, nkv, d, p, r)) for r in range(p)]
    for r, y in enumerate(parts):
        assert y.shape[1] == sum(seg)
        h = r * nkv // p
        np.testing.assert_array_equal(y[:, seg[0]:seg[0] + seg[1]], full[:, (nh + h) * d:(nh + h + 1) * d])
        np.testing.assert_array_equal(y[:, seg[0] + seg[1]:], full[:, (nh + nkv + h) * d:(nh + nkv + h + 1) * d])
    cat = O.concat(parts, seg)
    assert cat.shape[1] == (nh + 2 * p) * d
    np.testing.assert_array_equal(O.qkv_unreplicate(cat, nh, nkv, d, p), full)
    # without replication the concat already is the unsharded layout
    parts2 = [O.col_linear(x, *O.qkv_shard(wt["Wqkv"], wt["bqkv"], nh, nkv, d, 2, r)) for r in range(2)]
    np.testing.assert_array_equal(O.qkv_unreplicate(O.concat(parts2, O.qkv_segments(nh, nkv, d, 2)), nh, nkv, d, 2),
                                  full)
    # the layer chain over 8 shards with 2 KV heads equals the unsharded chain
    shape = I.LayerShape("t", hidden=hid, intermediate=24, n_heads=nh, n_kv_heads=nkv, head_dim=d, tp=p, seed=14)
    w = {k: I.as_numpy_f64(v) for k, v in {**I.attn_weights(shape), **I.ffn_weights(shape)}.items()}
    w.update(n_heads=nh, n_kv_heads=nkv, head_dim=d)
    got = O.layer_sharded(x, w, p)
    np.testing.assert_array_equal(got["qkv"], O.linear(x, w["Wqkv"], w["bqkv"]))
    assert O.rel_err(got["y"], O.layer_unsharded(x, w)) <= 1e-12


def _qkv(m, hq, hk, d, seed):
    return I.as_numpy_f64(I.activations(m, (hq + 2 * hk) * d, seed=seed))


def test_attention_uniform_scores_give_prefix_means():
    """K = 0: every allowed key scores the same, so O_i = mean(v_0..v_i) (causal) or the mean of all."""
    m, hq, hk, d = 6, 2, 1, 4
    qkv = _qkv(m, hq, hk, d, 61)
    qkv[:, hq * d:(hq + hk) * d] = 0.0
    v = qkv[:, (hq + hk) * d:]
    a = O.attention_core_shard(qkv, hq, hk, d, causal=True)
    prefix = np.cumsum(v, axis=0) / np.arange(1, m + 1)[:, None]
    for h in range(hq):
        np.testing.assert_allclose(a[:, h * d:(h + 1) * d], prefix, rtol=1e-14, atol=1e-15)
    a2 = O.attention_core_shard(qkv, hq, hk, d, causal=False)
    np.testing.assert_allclose(a2[:, :d], np.broadcast_to(v.mean(axis=0), (m, d)), rtol=1e-14, atol=1e-15)


def test_attention_first_causal_row_and_dominant_key():
    m, hq, hk, d = 5, 4, 2, 8
    qkv = _qkv(m, hq, hk, d, 62)
    a = O.attention_core_shard(qkv, hq, hk, d)
    for h, g in zip(range(hq), (0, 0, 1, 1)):   # consecutive query heads share a KV head
        assert O.kv_group_of(h, hq, hk) == g
        np.testing.assert_array_equal(a[0, h * d:(h + 1) * d], qkv[0, (hq + hk + g) * d:(hq + hk + g + 1) * d])
    # a key aligned with every query at a huge scale takes all the weight (non-causal)
    qkv2 = qkv.copy()
    qkv2[:, :hq * d] = 1.0
    qkv2[:, hq * d:(hq + hk) * d] = -1.0
    qkv2[3, hq * d:(hq + hk) * d] = 200.0
    a2 = O.attention_core_shard(qkv2, hq, hk, d, causal=False)
    for h, g in zip(range(hq), (0, 0, 1, 1)):
        np.testing.assert_allclose(a2[:, h * d:(h + 1) * d],
                                   np.broadcast_to(qkv2[3, (hq + hk + g) * d:(hq + hk + g + 1) * d], (m, d)), rtol=1e-12)


def test_attention_tiny_by_bruteforce():
    m, hq, hk, d = 4, 4, 2, 3
    qkv = _qkv(m, hq, hk, d, 63)
    a = O.attention_core_shard(qkv, hq, hk, d)
    for h in range(hq):
        g = h // (hq // hk)
        for i in range(m):
            sc = [math.fsum(qkv[i, h * d + t] * qkv[j, (hq + g) * d + t] for t in range(d)) / math.sqrt(d)
                  for j in range(i + 1)]
            mx = max(sc)
            w = [math.exp(c - mx) for c in sc]
            z = math.fsum(w)
            for t in range(d):
                o = math.fsum(w[j] * qkv[j, (hq + hk + g) * d + t] for j in range(i + 1)) / z
                assert abs(a[i, h * d + t] - o) <= 1e-13 * max(1.0, abs(o))


def test_attention_shards_equal_unsharded_heads():
    """Heads are independent: shard r's output is the unsharded attention's block of its heads."""
    m, nh, nkv, d, p = 7, 8, 2, 4, 2
    shape = I.LayerShape("t", hidden=16, n_heads=nh, n_kv_heads=nkv, head_dim=d, tp=p, seed=64)
    wt = {k: I.as_numpy_f64(v) for k, v in I.attn_weights(shape).items()}
    x = I.as_numpy_f64(I.activations(m, 16, seed=641))
    full = O.attention_core_shard(O.linear(x, wt["Wqkv"], wt["bqkv"]), nh, nkv, d)
    for r in range(p):
        w_r, b_r = O.qkv_shard(wt["Wqkv"], wt["bqkv"], nh, nkv, d, p, r)
        a_r = O.attention_core_shard(O.col_linear(x, w_r, b_r), nh // p, nkv // p, d)
        np.testing.assert_allclose(a_r, full[:, r * (nh // p) * d:(r + 1) * (nh // p) * d], rtol=1e-12, atol=1e-14)


def test_attention_decode_over_cache_equals_the_full_causal_pass():
    """Causality: a token's output does not depend on later tokens, so feeding a sequence in
    chunks through the cache gives the rows of one causal pass over the whole sequence; the
    cache ends up holding exactly the sequence's K and V columns."""
    m, hq, hk, d = 11, 4, 2, 8
    qkv = _qkv(m, hq, hk, d, 65)
    full = O.attention_core_shard(qkv, hq, hk, d, causal=True)
    kc = np.zeros((0, hk * d))
    vc = np.zeros((0, hk * d))
    t = 0
    for chunk in (4, 1, 1, 5):
        a, kc, vc = O.attention_decode_shard(qkv[t:t + chunk], kc, vc, hq, hk, d)
        np.testing.assert_allclose(a, full[t:t + chunk], rtol=1e-12, atol=1e-14)
        t += chunk
    np.testing.assert_array_equal(kc, qkv[:, hq * d:(hq + hk) * d])
    np.testing.assert_array_equal(vc, qkv[:, (hq + hk) * d:])


def test_attention_decode_single_token_by_bruteforce():
    """One new token over a 3-row cache: explicit fsum loops over its 4 allowed keys."""
    hq, hk, d, t = 2, 1, 3, 3
    qkv = _qkv(t + 1, hq, hk, d, 66)
    kc, vc = qkv[:t, hq * d:(hq + hk) * d], qkv[:t, (hq + hk) * d:]
    a, _, _ = O.attention_decode_shard(qkv[t:], kc, vc, hq, hk, d)
    for h in range(hq):
        sc = [math.fsum(qkv[t, h * d + x] * qkv[j, hq * d + x] for x in range(d)) / math.sqrt(d) for j in range(t + 1)]
        mx = max(sc)
        w = [math.exp(c - mx) for c in sc]
        z = math.fsum(w)
        for x in range(d):
            o = math.fsum(w[j] * qkv[j, (hq + hk) * d + x] for j in range(t + 1)) / z
            assert abs(a[0, h * d + x] - o) <= 1e-13 * max(1.0, abs(o))


def test_indivisible_sizes_are_rejected():
    w = np.zeros((10, 9))
    with pytest.raises(ValueError):
        O.col_shard(w, None, 3, 0)
    with pytest.raises(ValueError):
        O.row_shard(w, 2, 0)
    with pytest.raises(ValueError):
        O.qkv_rows(64, 8, 128, 3, 0)


@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_mlp_pairing_sum_of_partials_equals_unsharded(p):
    """Column then row: the intermediate is never combined; one sum at the end."""
    h, i, m = 32, 64, 5
    shape = I.LayerShape("t", hidden=h, intermediate=i, tp=p, seed=7)
    wt = {k: I.as_numpy_f64(v) for k, v in I.ffn_weights(shape).items()}
    x = I.as_numpy_f64(I.activations(m, h, seed=71))
    ref = O.mlp(x, wt["Wg"], wt["Wu"], wt["Wd"], wt["bg"], wt["bu"], wt["bd"])
    shards = O.mlp_shards(x, wt["Wg"], wt["Wu"], wt["Wd"], p, wt["bg"], wt["bu"])
    y = O.combine_sum([pr for _, pr in shards], wt["bd"])
    assert O.rel_err(y, ref) <= 1e-13
    h_full = O.swiglu(O.linear(x, wt["Wg"], wt["bg"]), O.linear(x, wt["Wu"], wt["bu"]))
    np.testing.assert_array_equal(O.concat([h_r for h_r, _ in shards]), h_full)


def test_mlp_tiny_by_bruteforce():
    h, i, m, p = 6, 8, 2, 2
    shape = I.LayerShape("t", hidden=h, intermediate=i, tp=p, seed=8)
    wt = {k: I.as_numpy_f64(v) for k, v in I.ffn_weights(shape).items()}
    x = I.as_numpy_f64(I.activations(m, h, seed=81))
    g = O.linear_fsum(x, wt["Wg"], wt["bg"])
    u = O.linear_fsum(x, wt["Wu"], wt["bu"])
    hh = np.array([[gv / (1.0 + math.exp(-gv)) * uv for gv, uv in zip(gr, ur)] for gr, ur in zip(g, u)])
    y_bf = O.linear_fsum(hh, wt["Wd"], wt["bd"])
    y = O.mlp(x, wt["Wg"], wt["Wu"], wt["Wd"], wt["bg"], wt["bu"], wt["bd"])
    np.testing.assert_allclose(y, y_bf, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("p", [2, 4])
def test_gelu_ffn_pairing_sum_of_partials_equals_unsharded(p):
    """The listing's FFN: column layer, GELU, row layer; one sum and the bias at the end."""
    h, i, m = 32, 64, 4
    shape = I.LayerShape("t", hidden=h, intermediate=i, tp=p, seed=9)
    wt = {k: I.as_numpy_f64(v) for k, v in I.gelu_ffn_weights(shape).items()}
    x = I.as_numpy_f64(I.activations(m, h, seed=91))
    ref = O.ffn_gelu(x, wt["W1"], wt["W2"], wt["b1"], wt["b2"])
    shards = O.ffn_gelu_shards(x, wt["W1"], wt["W2"], p, wt["b1"])
    y = O.combine_sum([pr for _, pr in shards], wt["b2"])
    assert O.rel_err(y, ref) <= 1e-13
    np.testing.assert_array_equal(O.concat([h_r for h_r, _ in shards]), O.gelu(O.linear(x, wt["W1"], wt["b1"])))


def test_gelu_ffn_tiny_by_bruteforce():
    h, i, m = 6, 8, 2
    shape = I.LayerShape("t", hidden=h, intermediate=i, tp=2, seed=10)
    wt = {k: I.as_numpy_f64(v) for k, v in I.gelu_ffn_weights(shape).items()}
    x = I.as_numpy_f64(I.activations(m, h, seed=101))
    a = O.linear_fsum(x, wt["W1"], wt["b1"])
    hh = np.array([[0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in row] for row in a])
    y_bf = O.linear_fsum(hh, wt["W2"], wt["b2"])
    y = O.ffn_gelu(x, wt["W1"], wt["W2"], wt["b1"], wt["b2"])
    np.testing.assert_allclose(y, y_bf, rtol=1e-12, atol=1e-14)


def test_qkv_head_split_concat_and_one_hot():
    """Parity unpinned by the pages: self-consistency of the head layout only."""
    nh, nkv, d, hid, p = 8, 2, 4, 16, 2
    shape = I.LayerShape("t", hidden=hid, n_heads=nh, n_kv_heads=nkv, head_dim=d, tp=p, seed=9)
    wt = {k: I.as_numpy_f64(v) for k, v in I.attn_weights(shape).items()}
    x = I.as_numpy_f64(I.activations(3, hid, seed=91))
    parts = []
    for r in range(p):
        w_r, b_r = O.qkv_shard(wt["Wqkv"], wt["bqkv"], nh, nkv, d, p, r)
        assert w_r.shape == ((nh // p + 2 * nkv // p) * d, hid)
        parts.append(O.col_linear(x, w_r, b_r))
    full = O.linear(x, wt["Wqkv"], wt["bqkv"])
    np.testing.assert_array_equal(O.concat(parts, O.qkv_segments(nh, nkv, d, p)), full)
    # One-hot input: shard r's K segment holds exactly the weight column of its own KV head.
    for r in range(p):
        w_r, _ = O.qkv_shard(wt["Wqkv"], None, nh, nkv, d, p, r)
        e = np.zeros((1, hid))
        e[0, 3] = 1.0
        y = O.col_linear(e, w_r)[0]
        k_rows = wt["Wqkv"][nh * d + r * (nkv // p) * d: nh * d + (r + 1) * (nkv // p) * d, 3]
        np.testing.assert_array_equal(y[nh // p * d: nh // p * d + nkv // p * d], k_rows)


def test_layer_sharded_equals_unsharded_small():
    nh, nkv, d, hid, inter, p = 8, 4, 4, 32, 48, 4
    shape = I.LayerShape("t", hidden=hid, intermediate=inter, n_heads=nh, n_kv_heads=nkv,
                         head_dim=d, tp=p, seed=10)
    w = {k: I.as_numpy_f64(v) for k, v in {**I.attn_weights(shape), **I.ffn_weights(shape)}.items()}
    w.update(n_heads=nh, n_kv_heads=nkv, head_dim=d)
    x = I.as_numpy_f64(I.activations(6, hid, seed=101))
    ref = O.layer_unsharded(x, w)
    got = O.layer_sharded(x, w, p)
    assert O.rel_err(got["y"], ref) <= 1e-12
    np.testing.assert_array_equal(got["qkv"], O.linear(x, w["Wqkv"], w["bqkv"]))


def test_rel_err_definition():
    assert O.rel_err(np.array([1.0, -3.0]), np.array([1.0, -2.0])) == 0.5
    assert O.rel_err(np.zeros(3), np.zeros(3)) == 0.0
    assert O.rel_err(np.array([0.1]), np.zeros(1)) == pytest.approx(0.1)
