"""CPU fp64 oracle for one GPU's tensor-parallel shard of a transformer layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library and
its Python binding) never calls it, and it shares no code with that path.

Everything here is plain numpy float64 on the CPU, written so that each function
can be checked by eye against the passage it cites:

  [P3] "Understanding Tensor Parallelism for Multi-GPU LLM Serving" (DevBytes),
       section "How Tensor Parallelism Works Under the Hood" and the
       ColumnParallelLinear / RowParallelLinear listing of section
       "Implementing Tensor Parallelism with Hugging Face Accelerate".
  [P4] "What is tensor parallelism?" (tecyfy), section "How a layer is split".
  [P5] "Tensor parallel serving" (Learn AI), the simulation script of section
       "Simulating the split, and proving it is correct", its "Line-by-line
       walkthrough", "Common mistakes", "Try it yourself" and the researcher
       section "Column-parallel and row-parallel layers, paired".

Inputs are arrays of stored values (bf16 or fp32); they are widened exactly to
float64 and every intermediate stays float64 and unrounded.

Conventions (readings where the pages leave a step open):
  * A weight is stored [out_features, in_features] row-major, as the listing
    stores it; the pages' Y = XW is therefore computed as X @ W^T (+ b), the
    form the simulation script uses.
  * Shard r of p owns the contiguous block [r*n/p, (r+1)*n/p) of the split
    dimension; concat and sum run in rank order.
  * SwiGLU is silu(X Wg^T + bg) * (X Wu^T + bu), silu(z) = z / (1 + exp(-z)).
    The pages never define it (they show GELU); this is the usual gated form.
  * Head split of a fused QKV weight: shard r owns Q heads
    [r*H/p, (r+1)*H/p) and KV heads [r*G/p, (r+1)*G/p) (GQA is not on the
    pages; this is the plain reading of "different attention heads go to
    different GPUs" with the TP size dividing the head counts).

Parity status per function (what pins it, beside itself):
  linear, col_shard, row_shard, concat, combine_sum:  pinned (printed toy
      output, brute-force fsum, closed-form special cases, page invariants).
  silu / swiglu:  pinned by closed forms of the definition; the choice of
      SwiGLU over GELU is a reading.
  gelu / ffn_gelu:  gelu pinned by closed forms (odd-part identity, tabulated
      normal CDF values); the FFN by the sharded-equals-unsharded invariant.
  qkv head layout / attention stand-in (A := Q):  parity unpinned by the
      pages (self-consistency invariants only).
  kv_heads_of / qkv_segments / qkv_unreplicate with more shards than KV heads
      (replication):  a reading, parity unpinned by the pages (self-consistency
      invariants only: every replica's K/V segment equals its head's columns of the
      unsharded QKV, and the de-replicated concat equals the unsharded QKV).
  blocks_of / row_shard_uneven:  pinned by the uneven-split invariant of [P5]
      "Try it yourself" and brute force.
  attention_core_shard:  the core is not on the pages (a reading: causal,
      grouped-query scaled dot-product attention); pinned by closed forms of
      softmax attention (uniform scores give the prefix mean of V, the first
      causal row is v_0, a dominant score selects its value row) and brute force.
"""
from __future__ import annotations

import math

import numpy as np


def f64(a) -> np.ndarray:
    """Exact widening of stored values to float64."""
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# The linear layer Y = XW  ([P3] "How Tensor Parallelism Works Under the Hood";
# [P5] simulation script: full_output = x @ W.T + b)
# ---------------------------------------------------------------------------

def linear(x, w, b=None) -> np.ndarray:
    """Y[m, n] = sum_k X[m, k] * W[n, k] (+ b[n]), W stored [out, in]."""
    y = f64(x) @ f64(w).T
    if b is not None:
        y = y + f64(b)[None, :]
    return y


def linear_fsum(x, w, b=None) -> np.ndarray:
    """The same definition with explicit loops and an exactly rounded sum.

    Products of two bf16 or fp32 values are exact in float64, so math.fsum
    returns the correctly rounded dot product.  For tiny inputs only.
    """
    x, w = f64(x), f64(w)
    m_count, k_count = x.shape
    n_count = w.shape[0]
    y = np.empty((m_count, n_count))
    for m in range(m_count):
        for n in range(n_count):
            terms = [x[m, k] * w[n, k] for k in range(k_count)]
            if b is not None:
                terms.append(float(f64(b)[n]))
            y[m, n] = math.fsum(terms)
    return y


def linear_entry(x_row, w_row, b_n=None) -> float:
    """One output entry by fsum: for spot checks of large shapes."""
    terms = list(f64(x_row) * f64(w_row))
    if b_n is not None:
        terms.append(float(b_n))
    return math.fsum(terms)


# ---------------------------------------------------------------------------
# Sharding ([P3] listing: out_features // world_size rows per rank for the
# column layer, in_features // world_size inputs for the row layer, both
# asserted divisible; [P5] W[:split], W[split:])
# ---------------------------------------------------------------------------

def _block(n: int, p: int, r: int) -> slice:
    if p <= 0 or n % p != 0:
        raise ValueError(f"size {n} is not divisible by tensor_parallel_size {p}")
    if not 0 <= r < p:
        raise ValueError(f"rank {r} outside [0, {p})")
    step = n // p
    return slice(r * step, (r + 1) * step)


def col_shard(w, b, p: int, r: int):
    """Column-parallel shard r: the block of output rows W[r*N/p:(r+1)*N/p, :] and b likewise."""
    s = _block(np.shape(w)[0], p, r)
    return f64(w)[s, :], (None if b is None else f64(b)[s])


def col_shard_uneven(w, b, widths):
    """Column split into consecutive blocks of the given widths ([P5] "Try it yourself")."""
    out, start = [], 0
    for width in widths:
        out.append((f64(w)[start:start + width, :],
                    None if b is None else f64(b)[start:start + width]))
        start += width
    if start != np.shape(w)[0]:
        raise ValueError("widths do not cover the output features")
    return out


def blocks_of(n: int, widths):
    """Consecutive blocks of the given widths covering n ([P5] "Try it yourself": an uneven
    split still matches exactly)."""
    out, start = [], 0
    for width in widths:
        if width <= 0:
            raise ValueError("block widths must be positive")
        out.append(slice(start, start + width))
        start += width
    if start != n:
        raise ValueError("widths do not cover the dimension")
    return out


def row_shard_uneven(w, widths):
    """Row split into consecutive input-column blocks of the given widths."""
    return [f64(w)[:, s] for s in blocks_of(np.shape(w)[1], widths)]


def input_slices_uneven(x, widths):
    """The matching column blocks of the row layer's input."""
    return [f64(x)[:, s] for s in blocks_of(np.shape(x)[1], widths)]


def row_shard(w, p: int, r: int) -> np.ndarray:
    """Row-parallel shard r: the block of input columns W[:, r*K/p:(r+1)*K/p]."""
    s = _block(np.shape(w)[1], p, r)
    return f64(w)[:, s]


def input_slice(x, p: int, r: int) -> np.ndarray:
    """x[..., r*K/p:(r+1)*K/p], the slice the row layer takes by rank ([P3] RowParallelLinear.forward)."""
    s = _block(np.shape(x)[1], p, r)
    return f64(x)[:, s]


# ---------------------------------------------------------------------------
# Per-shard products
# ---------------------------------------------------------------------------

def col_linear(x, w_r, b_r=None) -> np.ndarray:
    """Y_r = X W_r (+ b_r): full, replicated input; a slice of the output ([P3], [P5])."""
    return linear(x, w_r, b_r)


def row_partial(x_r, w_r) -> np.ndarray:
    """P_r = X_r W_r with no bias: a partial sum of the full output ([P3])."""
    return linear(x_r, w_r, None)


# ---------------------------------------------------------------------------
# Combines ([P5] torch.cat([...], dim=-1); [P3] all_reduce(SUM) then + bias;
# [P5] "Common mistakes": row-parallel combines by summing, not concatenating)
# ---------------------------------------------------------------------------

def concat(shards, seg_widths=None) -> np.ndarray:
    """Concatenate per-shard outputs along the feature axis, in rank order.

    With seg_widths = (w_0, ..., w_{s-1}) each shard holds s segments side by
    side; segment j of every shard is gathered into output block j, shards in
    rank order inside the block (used for the fused Q|K|V output).
    """
    shards = [f64(s) for s in shards]
    if seg_widths is None:
        return np.concatenate(shards, axis=-1)
    blocks = []
    start = 0
    for width in seg_widths:
        blocks.append(np.concatenate([s[:, start:start + width] for s in shards], axis=-1))
        start += width
    return np.concatenate(blocks, axis=-1)


def combine_sum(partials, b=None) -> np.ndarray:
    """Y = sum_r P_r, ranks ascending, then + b once."""
    acc = np.zeros_like(f64(partials[0]))
    for p_r in partials:
        acc = acc + f64(p_r)
    if b is not None:
        acc = acc + f64(b)[None, :]
    return acc


# ---------------------------------------------------------------------------
# Activation between the paired layers
# ---------------------------------------------------------------------------

def silu(z) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(g, u) -> np.ndarray:
    """H = silu(G) * U, elementwise."""
    return silu(g) * f64(u)


def gelu(z) -> np.ndarray:
    """The exact (erf) GELU that the listing's FFN applies between its column and row
    layers ([P3] "Implementing Tensor Parallelism with Hugging Face Accelerate",
    torch.nn.functional.gelu with its default form): gelu(z) = z * Phi(z), with
    Phi the standard normal CDF, Phi(z) = (1 + erf(z / sqrt(2))) / 2."""
    z = f64(z)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def _erf(z) -> np.ndarray:
    try:
        from scipy.special import erf
        return erf(z)
    except ImportError:  # pragma: no cover - scipy is present in this image
        return np.vectorize(math.erf)(z)


# ---------------------------------------------------------------------------
# Paired column -> row MLP ([P3] "How Tensor Parallelism Works Under the Hood":
# first layer column-parallel, second row-parallel; [P5] researcher section:
# the intermediate between them is never communicated)
# ---------------------------------------------------------------------------

def mlp(x, wg, wu, wd, bg=None, bu=None, bd=None):
    """Unsharded SwiGLU MLP: Y = (silu(X Wg^T + bg) * (X Wu^T + bu)) Wd^T + bd."""
    h = swiglu(linear(x, wg, bg), linear(x, wu, bu))
    return linear(h, wd, bd)


def mlp_shard(x, wg_r, wu_r, wd_r, bg_r=None, bu_r=None):
    """Shard r of the MLP: H_r from the column pair, P_r = H_r Wd_r^T (no bias)."""
    h_r = swiglu(col_linear(x, wg_r, bg_r), col_linear(x, wu_r, bu_r))
    return h_r, row_partial(h_r, wd_r)


def mlp_shards(x, wg, wu, wd, p, bg=None, bu=None):
    """All p shards, from slices of the unsharded weights."""
    out = []
    for r in range(p):
        wg_r, bg_r = col_shard(wg, bg, p, r)
        wu_r, bu_r = col_shard(wu, bu, p, r)
        wd_r = row_shard(wd, p, r)
        out.append(mlp_shard(x, wg_r, wu_r, wd_r, bg_r, bu_r))
    return out


# The listing's own FFN ([P3] "Implementing Tensor Parallelism with Hugging Face
# Accelerate": a ColumnParallelLinear 4096 -> 11008, GELU, a RowParallelLinear
# 11008 -> 4096 whose bias is added once after the reduction)

def ffn_gelu(x, w1, w2, b1=None, b2=None):
    """Unsharded: Y = gelu(X W1^T + b1) W2^T + b2."""
    return linear(gelu(linear(x, w1, b1)), w2, b2)


def ffn_gelu_shard(x, w1_r, w2_r, b1_r=None):
    """Shard r: H_r = gelu(X W1_r^T + b1_r) (column), P_r = H_r W2_r^T (row partial, no bias)."""
    h_r = gelu(col_linear(x, w1_r, b1_r))
    return h_r, row_partial(h_r, w2_r)


def ffn_gelu_shards(x, w1, w2, p, b1=None):
    """All p shards, from slices of the unsharded weights."""
    out = []
    for r in range(p):
        w1_r, b1_r = col_shard(w1, b1, p, r)
        out.append(ffn_gelu_shard(x, w1_r, row_shard(w2, p, r), b1_r))
    return out


# ---------------------------------------------------------------------------
# Head-split attention projections ([P4] "How a layer is split": heads go to
# different GPUs; the TP size divides the heads; [P5] one all-reduce per
# attention block)
# ---------------------------------------------------------------------------

def kv_heads_of(n_kv_heads, p, r):
    """KV heads held by shard r: the block [r*G/p, (r+1)*G/p) when p divides G. When there
    are more shards than KV heads and p is a multiple of G (a reading: the pages only say
    the TP size divides the heads), each KV head is replicated on p/G consecutive shards
    and shard r holds head floor(r*G/p)."""
    if not 0 <= r < p:
        raise ValueError(f"rank {r} outside [0, {p})")
    if n_kv_heads % p == 0:
        hk = n_kv_heads // p
        return list(range(r * hk, (r + 1) * hk))
    if p % n_kv_heads == 0:
        return [r * n_kv_heads // p]
    raise ValueError("tensor_parallel_size must divide the KV heads or be a multiple of them")


def qkv_rows(n_heads, n_kv_heads, head_dim, p, r):
    """Row indices of the fused [Wq; Wk; Wv] weight owned by shard r, in order Q | K | V."""
    if n_heads % p:
        raise ValueError("tensor_parallel_size must divide the head counts")
    hq, d = n_heads // p, head_dim
    q = np.arange(r * hq * d, (r + 1) * hq * d)
    kv = kv_heads_of(n_kv_heads, p, r)
    k = np.concatenate([np.arange((n_heads + h) * d, (n_heads + h + 1) * d) for h in kv])
    v = np.concatenate([np.arange((n_heads + n_kv_heads + h) * d, (n_heads + n_kv_heads + h + 1) * d) for h in kv])
    return np.concatenate([q, k, v])


def qkv_shard(wqkv, bqkv, n_heads, n_kv_heads, head_dim, p, r):
    rows = qkv_rows(n_heads, n_kv_heads, head_dim, p, r)
    return f64(wqkv)[rows, :], (None if bqkv is None else f64(bqkv)[rows])


def qkv_segments(n_heads, n_kv_heads, head_dim, p):
    """Per-shard segment widths of the fused output: (Q, K, V) = (Hq/p heads, the shard's KV
    heads, the shard's KV heads), each head head_dim wide. A shard holds G/p KV heads when p
    divides G, and the one replicated KV head when p is a multiple of G (kv_heads_of)."""
    if n_heads % p:
        raise ValueError("tensor_parallel_size must divide the head counts")
    hk = len(kv_heads_of(n_kv_heads, p, 0))
    return (n_heads // p * head_dim, hk * head_dim, hk * head_dim)


def qkv_unreplicate(qkv_cat, n_heads, n_kv_heads, head_dim, p):
    """The unsharded [Q | K | V] columns from the segment concat of all p shards' QKV outputs.

    When p divides G the concat already is the unsharded layout. When KV heads are
    replicated (p a multiple of G) the concat's K and V blocks hold p heads, head
    floor(r*G/p) at block r, so KV head h is taken from its first holder, shard h*p/G.
    Index selection only."""
    qkv_cat = f64(qkv_cat)
    if n_kv_heads % p == 0:
        return qkv_cat
    d, nq = head_dim, n_heads * head_dim
    first = [h * p // n_kv_heads for h in range(n_kv_heads)]
    k = [qkv_cat[:, nq + r * d:nq + (r + 1) * d] for r in first]
    v = [qkv_cat[:, nq + (p + r) * d:nq + (p + r + 1) * d] for r in first]
    return np.concatenate([qkv_cat[:, :nq]] + k + v, axis=-1)


def attn_proj_shard(x, wqkv_r, bqkv_r, a_r, wo_r):
    """QKV_r = X Wqkv_r^T + bqkv_r (column); P_r = A_r Wo_r^T (row partial)."""
    qkv_r = None if wqkv_r is None else col_linear(x, wqkv_r, bqkv_r)
    p_r = None if wo_r is None else row_partial(a_r, wo_r)
    return qkv_r, p_r


# ---------------------------------------------------------------------------
# Head-local attention core between QKV_r and the O projection.  Heads go to
# different GPUs ([P4] "How a layer is split"), so a shard attends with its own
# heads only and needs no exchange.  The core itself is not on the pages; this is
# the plain reading: scaled dot-product attention over the M tokens of one
# sequence, causal (a decoder), grouped-query (query head h of the shard uses its
# KV head h // (hq / hk)).
# ---------------------------------------------------------------------------

def kv_group_of(h, hq, hk):
    """The shard-local KV head of shard-local query head h."""
    return h // (hq // hk)


def attention_core_shard(qkv_r, hq, hk, d, causal=True):
    """A_r[M, hq*d] from QKV_r[M, (hq + 2 hk) d] (segments Q | K | V): for each query head h,
    O_h = softmax(Q_h K_g^T / sqrt(d), masked to keys j <= i when causal) V_g, g = kv_group_of(h)."""
    qkv_r = f64(qkv_r)
    m = qkv_r.shape[0]
    out = np.empty((m, hq * d))
    for h in range(hq):
        g = kv_group_of(h, hq, hk)
        q = qkv_r[:, h * d:(h + 1) * d]
        k = qkv_r[:, (hq + g) * d:(hq + g + 1) * d]
        v = qkv_r[:, (hq + hk + g) * d:(hq + hk + g + 1) * d]
        s = (q @ k.T) / math.sqrt(d)
        if causal:
            s = np.where(np.tril(np.ones((m, m), dtype=bool)), s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        out[:, h * d:(h + 1) * d] = (e / e.sum(axis=1, keepdims=True)) @ v
    return out


def attention_decode_shard(qkv_new, k_cache, v_cache, hq, hk, d):
    """Decode step over a KV cache: the new tokens' projections qkv_new[M, (hq + 2 hk) d] sit at
    positions T .. T + M - 1 after the T cached rows k_cache, v_cache [T, hk d] (KV head g at
    columns g*d). Token i sees keys 0 .. T + i: the cache and the new tokens up to itself.
    Returns (A[M, hq*d], the caches with the new rows appended)."""
    qkv_new, k_cache, v_cache = f64(qkv_new), f64(k_cache), f64(v_cache)
    m, t = qkv_new.shape[0], k_cache.shape[0]
    k_all = np.concatenate([k_cache, qkv_new[:, hq * d:(hq + hk) * d]], axis=0)
    v_all = np.concatenate([v_cache, qkv_new[:, (hq + hk) * d:(hq + 2 * hk) * d]], axis=0)
    out = np.empty((m, hq * d))
    for h in range(hq):
        g = kv_group_of(h, hq, hk)
        q = qkv_new[:, h * d:(h + 1) * d]
        k = k_all[:, g * d:(g + 1) * d]
        v = v_all[:, g * d:(g + 1) * d]
        s = (q @ k.T) / math.sqrt(d)
        allowed = np.arange(t + m)[None, :] <= (t + np.arange(m))[:, None]
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        out[:, h * d:(h + 1) * d] = (e / e.sum(axis=1, keepdims=True)) @ v
    return out, k_all, v_all


# ---------------------------------------------------------------------------
# Full layer chain with the attention-core stand-in A := Q (a reading: the core
# is not on the pages).  X -> QKV -> A := Q -> Y1 = sum_r O-partials + bo
#   -> Y = sum_r MLP-partials(Y1) + bd.   No residual, no norm.
# ---------------------------------------------------------------------------

def layer_unsharded(x, w):
    """w: dict with Wqkv, bqkv, Wo, bo, Wg, bg, Wu, bu, Wd, bd and n_heads, n_kv_heads, head_dim."""
    nq = w["n_heads"] * w["head_dim"]
    qkv = linear(x, w["Wqkv"], w.get("bqkv"))
    a = qkv[:, :nq]
    y1 = linear(a, w["Wo"], w.get("bo"))
    return mlp(y1, w["Wg"], w["Wu"], w["Wd"], w.get("bg"), w.get("bu"), w.get("bd"))


def layer_sharded(x, w, p):
    """The same chain computed shard by shard and combined (column, row, sum, concat)."""
    nh, nkv, d = w["n_heads"], w["n_kv_heads"], w["head_dim"]
    qkv_parts, o_parts = [], []
    for r in range(p):
        wqkv_r, bqkv_r = qkv_shard(w["Wqkv"], w.get("bqkv"), nh, nkv, d, p, r)
        qkv_r = col_linear(x, wqkv_r, bqkv_r)
        a_r = qkv_r[:, : nh // p * d]
        o_parts.append(row_partial(a_r, row_shard(w["Wo"], p, r)))
        qkv_parts.append(qkv_r)
    y1 = combine_sum(o_parts, w.get("bo"))
    mlp_parts = mlp_shards(y1, w["Wg"], w["Wu"], w["Wd"], p, w.get("bg"), w.get("bu"))
    y = combine_sum([pr for _, pr in mlp_parts], w.get("bd"))
    qkv = qkv_unreplicate(concat(qkv_parts, qkv_segments(nh, nkv, d, p)), nh, nkv, d, p)
    h = concat([h_r for h_r, _ in mlp_parts])
    return {"qkv": qkv, "y1": y1, "h": h, "y": y}


# ---------------------------------------------------------------------------
# Error metric: e = max|y - y_ref| / max|y_ref| (absolute when y_ref is all zero)
# ---------------------------------------------------------------------------

def rel_err(y, y_ref) -> float:
    y, y_ref = f64(y), f64(y_ref)
    if y.shape != y_ref.shape:
        raise ValueError(f"shape {y.shape} != {y_ref.shape}")
    if y.size == 0:
        return 0.0
    num = float(np.max(np.abs(y - y_ref)))
    den = float(np.max(np.abs(y_ref)))
    return num / den if den > 0 else num
