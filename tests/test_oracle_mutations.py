"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Each mutation replaces one oracle function with a wrong variant; the listed pin
tests must then fail.  This shows the pins are sensitive to dropped terms,
wrong signs or indices, and transposed or misplaced operands.
"""
import numpy as np
import pytest

import oracle
import oracle.tp_oracle as T
import test_oracle_pins as P


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(T, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _linear_no_bias(x, w, b=None):
    return T.f64(x) @ T.f64(w).T


def _linear_bias_twice(x, w, b=None):
    y = T.f64(x) @ T.f64(w).T
    return y if b is None else y + 2 * T.f64(b)[None, :]


def _silu_wrong_sign(z):
    z = T.f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(z))


def _silu_sigmoid_only(z):
    z = T.f64(z)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def _gelu_tanh_approximation(z):
    z = T.f64(z)
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def _gelu_erf_unscaled(z):
    z = T.f64(z)
    return 0.5 * z * (1.0 + T._erf(z))


def _combine_sum_bias_each(partials, b=None):
    acc = np.zeros_like(T.f64(partials[0]))
    for p_r in partials:
        acc = acc + T.f64(p_r) + (0 if b is None else T.f64(b)[None, :])
    return acc


def _combine_sum_drop_last(partials, b=None):
    acc = np.zeros_like(T.f64(partials[0]))
    for p_r in partials[:-1]:
        acc = acc + T.f64(p_r)
    return acc if b is None else acc + T.f64(b)[None, :]


def _col_shard_off_by_one(w, b, p, r):
    n = np.shape(w)[0]
    step = n // p
    s = slice(r * step + (1 if r else 0), (r + 1) * step + (1 if r and (r + 1) * step < n else 0))
    return T.f64(w)[s, :], (None if b is None else T.f64(b)[s])


def _row_shard_wrong_axis(w, p, r):
    n = np.shape(w)[0]
    step = n // p
    return T.f64(w)[r * step:(r + 1) * step, :]


def _concat_reversed(shards, seg_widths=None):
    return np.concatenate([T.f64(s) for s in shards[::-1]], axis=-1)


def _qkv_rows_shared_kv(n_heads, n_kv_heads, head_dim, p, r):
    hq, hk, d = n_heads // p, n_kv_heads // p, head_dim
    q = np.arange(r * hq * d, (r + 1) * hq * d)
    k = np.arange(n_heads * d, n_heads * d + hk * d)            # always KV head block 0
    v = np.arange((n_heads + n_kv_heads) * d, (n_heads + n_kv_heads) * d + hk * d)
    return np.concatenate([q, k, v])


def _kv_heads_of_no_replication(n_kv_heads, p, r):
    if n_kv_heads % p == 0:
        hk = n_kv_heads // p
        return list(range(r * hk, (r + 1) * hk))
    return [r % n_kv_heads]          # round-robin instead of consecutive blocks


def _qkv_segments_floor(n_heads, n_kv_heads, head_dim, p):
    return (n_heads // p * head_dim, n_kv_heads // p * head_dim, n_kv_heads // p * head_dim)


def _qkv_unreplicate_ignores_replicas(qkv_cat, n_heads, n_kv_heads, head_dim, p):
    """Takes the first G K/V blocks of the concat as if no head were replicated."""
    qkv_cat = T.f64(qkv_cat)
    d, nq = head_dim, n_heads * head_dim
    blocks = p if n_kv_heads % p else n_kv_heads
    k = qkv_cat[:, nq:nq + n_kv_heads * d]
    v = qkv_cat[:, nq + blocks * d:nq + (blocks + n_kv_heads) * d]
    return np.concatenate([qkv_cat[:, :nq], k, v], axis=-1)


def _kv_group_round_robin(h, hq, hk):
    return h % hk


def _attention_unscaled(qkv_r, hq, hk, d, causal=True):
    return _attn_variant(qkv_r, hq, hk, d, causal, 1.0, True)


def _attention_no_mask(qkv_r, hq, hk, d, causal=True):
    return _attn_variant(qkv_r, hq, hk, d, causal, 1.0 / np.sqrt(d), False)


def _attn_variant(qkv_r, hq, hk, d, causal, scale, mask):
    qkv_r = T.f64(qkv_r)
    m = qkv_r.shape[0]
    out = np.empty((m, hq * d))
    for h in range(hq):
        g = h // (hq // hk)
        q, k = qkv_r[:, h * d:(h + 1) * d], qkv_r[:, (hq + g) * d:(hq + g + 1) * d]
        v = qkv_r[:, (hq + hk + g) * d:(hq + hk + g + 1) * d]
        s = (q @ k.T) * scale
        if causal and mask:
            s = np.where(np.tril(np.ones((m, m), dtype=bool)), s, -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h * d:(h + 1) * d] = (e / e.sum(axis=1, keepdims=True)) @ v
    return out


def _decode_excludes_self(qkv_new, k_cache, v_cache, hq, hk, d):
    return _decode_variant(qkv_new, k_cache, v_cache, hq, hk, d, 0)


def _decode_cache_only(qkv_new, k_cache, v_cache, hq, hk, d):
    return _decode_variant(qkv_new, k_cache, v_cache, hq, hk, d, None)


def _decode_variant(qkv_new, k_cache, v_cache, hq, hk, d, shift):
    """shift 0: token i sees keys j < T + i (the new tokens before it, not itself); None: only
    the cache (as if the new rows were appended after the attention). Key 0 always stays
    allowed so that no row is empty."""
    qkv_new, k_cache, v_cache = T.f64(qkv_new), T.f64(k_cache), T.f64(v_cache)
    m, t = qkv_new.shape[0], k_cache.shape[0]
    k_all = np.concatenate([k_cache, qkv_new[:, hq * d:(hq + hk) * d]], axis=0)
    v_all = np.concatenate([v_cache, qkv_new[:, (hq + hk) * d:(hq + 2 * hk) * d]], axis=0)
    keys = np.arange(t + m)[None, :]
    limit = (t + np.arange(m))[:, None] if shift is not None else np.full((m, 1), t)
    allowed = (keys < limit) | (keys == 0)
    out = np.zeros((m, hq * d))
    for h in range(hq):
        g = h // (hq // hk)
        q, k, v = qkv_new[:, h * d:(h + 1) * d], k_all[:, g * d:(g + 1) * d], v_all[:, g * d:(g + 1) * d]
        s = np.where(allowed, (q @ k.T) / np.sqrt(d), -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h * d:(h + 1) * d] = (e / e.sum(axis=1, keepdims=True)) @ v
    return out, k_all, v_all


MUTATIONS = [
    ("linear", _linear_no_bias, [P.test_toy_full_output_matches_printed_values]),
    ("linear", _linear_bias_twice, [P.test_toy_full_output_matches_printed_values,
                                    P.test_identity_weight_returns_input_plus_bias]),
    ("silu", _silu_wrong_sign, [P.test_silu_closed_forms, P.test_mlp_tiny_by_bruteforce]),
    ("silu", _silu_sigmoid_only, [P.test_silu_closed_forms, P.test_swiglu_special_cases]),
    ("gelu", _gelu_tanh_approximation, [P.test_gelu_closed_forms]),
    ("gelu", _gelu_erf_unscaled, [P.test_gelu_closed_forms, P.test_gelu_ffn_tiny_by_bruteforce]),
    ("combine_sum", _combine_sum_bias_each, [P.test_toy_row_split_sum_plus_bias_equals_unsharded]),
    ("combine_sum", _combine_sum_drop_last, [P.test_toy_row_split_sum_plus_bias_equals_unsharded]),
    ("col_shard", _col_shard_off_by_one, [P.test_toy_column_split_concat_matches_printed_values_and_is_exact]),
    ("row_shard", _row_shard_wrong_axis, [P.test_toy_row_split_sum_plus_bias_equals_unsharded]),
    ("concat", _concat_reversed, [P.test_toy_column_split_concat_matches_printed_values_and_is_exact]),
    ("qkv_rows", _qkv_rows_shared_kv, [P.test_qkv_head_split_concat_and_one_hot]),
    ("kv_group_of", _kv_group_round_robin, [P.test_attention_first_causal_row_and_dominant_key]),
    ("attention_core_shard", _attention_unscaled, [P.test_attention_tiny_by_bruteforce]),
    ("attention_core_shard", _attention_no_mask, [P.test_attention_uniform_scores_give_prefix_means,
                                                  P.test_attention_first_causal_row_and_dominant_key]),
    ("qkv_segments", _qkv_segments_floor, [P.test_qkv_segments_and_concat_with_replicated_kv_heads]),
    ("qkv_unreplicate", _qkv_unreplicate_ignores_replicas, [P.test_qkv_segments_and_concat_with_replicated_kv_heads]),
    ("kv_heads_of", _kv_heads_of_no_replication, [P.test_kv_heads_replicated_when_more_shards_than_kv_heads]),
    ("attention_decode_shard", _decode_excludes_self, [P.test_attention_decode_over_cache_equals_the_full_causal_pass,
                                                       P.test_attention_decode_single_token_by_bruteforce]),
    ("attention_decode_shard", _decode_cache_only, [P.test_attention_decode_over_cache_equals_the_full_causal_pass,
                                                    P.test_attention_decode_single_token_by_bruteforce]),
]


@pytest.mark.parametrize("name,fn,pins", MUTATIONS, ids=[f"{m[0]}-{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn, pins):
    _patch(monkeypatch, name, fn)
    for pin in pins:
        with pytest.raises((AssertionError, ValueError, IndexError)):
            pin()
