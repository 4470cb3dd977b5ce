"""Seeded synthetic inputs shared by the oracle side and the HIP side of the tests.

This module holds only the input recipe: shapes, seeds, value distributions and
the fp32 -> bf16 rounding of the draws. It contains none of the method's
arithmetic (no sharding, no products, no combines), so both sides can take their
inputs from here without sharing any computation.

Recipe (stated once, used everywhere):
  * every tensor is drawn in fp32 from a CPU ``torch.Generator`` with a fixed
    seed, in a fixed order, then (except for the toy) rounded to bf16 with
    round-to-nearest-even (``Tensor.to(torch.bfloat16)``); the bf16 values are
    the ground truth for both sides;
  * weights and biases ~ N(0, 0.02) (0.02 is the standard deviation),
    activations ~ N(0, 1);
  * the unsharded tensors are drawn first; shards are slices of them, taken by
    each side with its own code;
  * the toy layer uses the draw order of the simulation script on the
    "Tensor parallel serving" page (section "Simulating the split, and proving
    it is correct"): x = randn(1, 8), W = randn(6, 8), b = randn(6) after
    seeding 0, kept in fp32.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class LayerShape:
    """Sizes of one configuration.  ``tp`` is the tensor-parallel size p."""

    name: str
    hidden: int
    intermediate: int = 0
    n_heads: int = 0
    n_kv_heads: int = 0
    head_dim: int = 0
    tp: int = 1
    tokens: tuple = field(default_factory=tuple)
    seed: int = 0


# The five workloads, described by what they are.
TOY = LayerShape("toy-1x8-6x8-tp2", hidden=8, tp=2, tokens=(1,), seed=0)
LLAMA7B_FFN_TP2 = LayerShape("llama7b-ffn-tp2", hidden=4096, intermediate=11008, tp=2,
                             tokens=(1, 8, 64), seed=2)
LLAMA70B_FFN_TP4 = LayerShape("llama70b-ffn-tp4", hidden=8192, intermediate=28672, tp=4,
                              tokens=(1, 16, 64), seed=3)
LLAMA70B_ATTN_TP8 = LayerShape("llama70b-attnproj-tp8", hidden=8192, n_heads=64, n_kv_heads=8,
                               head_dim=128, tp=8, tokens=(1, 2048), seed=4)
LLAMA70B_LAYER_TP8 = LayerShape("llama70b-layer-prefill-tp8", hidden=8192, intermediate=28672,
                                n_heads=64, n_kv_heads=8, head_dim=128, tp=8, tokens=(4096,),
                                seed=5)

# The pages' own FFN: 4096 -> 11008 -> 4096 with GELU between the column and the
# row layer, batch 4, here at TP = 2.
PAGES_FFN_GELU_TP2 = LayerShape("pages-ffn-gelu-tp2", hidden=4096, intermediate=11008, tp=2,
                                tokens=(4,), seed=6)

CONFIGS = {s.name: s for s in (TOY, LLAMA7B_FFN_TP2, LLAMA70B_FFN_TP4, LLAMA70B_ATTN_TP8,
                                LLAMA70B_LAYER_TP8, PAGES_FFN_GELU_TP2)}


def _gen(seed: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(int(seed))


def to_bf16(t: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16, round to nearest even (torch's conversion)."""
    return t.to(torch.bfloat16)


def toy_layer():
    """x [1, 8], W [6, 8], b [6] in fp32, seed 0, the page's draw order."""
    g = _gen(0)
    x = torch.randn(1, 8, generator=g)
    w = torch.randn(6, 8, generator=g)
    b = torch.randn(6, generator=g)
    return x, w, b


def toy_layer_uneven(out_features: int = 9):
    """The page's exercise: same seed and order, OUT_FEATURES changed to 9."""
    g = _gen(0)
    x = torch.randn(1, 8, generator=g)
    w = torch.randn(out_features, 8, generator=g)
    b = torch.randn(out_features, generator=g)
    return x, w, b


def weight(rows: int, cols: int, seed: int, dtype=torch.bfloat16) -> torch.Tensor:
    """Weight matrix stored [rows=out_features, cols=in_features], N(0, 0.02)."""
    w = torch.randn(rows, cols, generator=_gen(seed)) * WEIGHT_STD
    return w.to(dtype) if dtype != torch.float32 else w


def bias(n: int, seed: int, dtype=torch.bfloat16) -> torch.Tensor:
    b = torch.randn(n, generator=_gen(seed)) * WEIGHT_STD
    return b.to(dtype) if dtype != torch.float32 else b


def activations(m: int, k: int, seed: int, dtype=torch.bfloat16) -> torch.Tensor:
    """Activations [m tokens, k features], N(0, 1)."""
    x = torch.randn(m, k, generator=_gen(seed))
    return x.to(dtype) if dtype != torch.float32 else x


def tensor_seed(cfg_seed: int, slot: int) -> int:
    """Distinct, fixed seed per tensor of a configuration (slot = which tensor)."""
    return cfg_seed * 100 + slot


def activation_seed(cfg_seed: int, m: int, slot: int = 0) -> int:
    """Activations of a configuration at m tokens: seed*1000 + m (+ slot offset)."""
    return cfg_seed * 1000 + m + 7919 * slot


# Tensor slots within a configuration (fixed so every caller draws the same values).
SLOT_WQKV, SLOT_BQKV, SLOT_WO, SLOT_BO = 1, 2, 3, 4
SLOT_WG, SLOT_BG, SLOT_WU, SLOT_BU, SLOT_WD, SLOT_BD = 5, 6, 7, 8, 9, 10
SLOT_W1, SLOT_B1, SLOT_W2, SLOT_B2 = 11, 12, 13, 14


def ffn_weights(shape: LayerShape, dtype=torch.bfloat16, with_bias: bool = True,
                hidden: int | None = None, intermediate: int | None = None):
    """Unsharded SwiGLU FFN weights: Wg, Wu [I, H]; Wd [H, I]; biases bg, bu [I], bd [H]."""
    h = hidden or shape.hidden
    i = intermediate or shape.intermediate
    s = shape.seed
    out = {
        "Wg": weight(i, h, tensor_seed(s, SLOT_WG), dtype),
        "Wu": weight(i, h, tensor_seed(s, SLOT_WU), dtype),
        "Wd": weight(h, i, tensor_seed(s, SLOT_WD), dtype),
    }
    if with_bias:
        out["bg"] = bias(i, tensor_seed(s, SLOT_BG), dtype)
        out["bu"] = bias(i, tensor_seed(s, SLOT_BU), dtype)
        out["bd"] = bias(h, tensor_seed(s, SLOT_BD), dtype)
    return out


def gelu_ffn_weights(shape: LayerShape, dtype=torch.bfloat16, with_bias: bool = True,
                     hidden: int | None = None, intermediate: int | None = None):
    """Unsharded GELU FFN weights: W1 [I, H] (column layer), W2 [H, I] (row layer); b1 [I], b2 [H]."""
    h = hidden or shape.hidden
    i = intermediate or shape.intermediate
    s = shape.seed
    out = {
        "W1": weight(i, h, tensor_seed(s, SLOT_W1), dtype),
        "W2": weight(h, i, tensor_seed(s, SLOT_W2), dtype),
    }
    if with_bias:
        out["b1"] = bias(i, tensor_seed(s, SLOT_B1), dtype)
        out["b2"] = bias(h, tensor_seed(s, SLOT_B2), dtype)
    return out


def attn_weights(shape: LayerShape, dtype=torch.bfloat16, with_bias: bool = True,
                 hidden: int | None = None, n_heads: int | None = None,
                 n_kv_heads: int | None = None, head_dim: int | None = None):
    """Unsharded attention projections.

    Wqkv is stored as the row blocks [Wq (n_heads*d rows); Wk (n_kv*d); Wv (n_kv*d)],
    each [*, hidden]; Wo is [hidden, n_heads*d].
    """
    h = hidden or shape.hidden
    nh = n_heads or shape.n_heads
    nkv = n_kv_heads or shape.n_kv_heads
    d = head_dim or shape.head_dim
    s = shape.seed
    rows = (nh + 2 * nkv) * d
    out = {
        "Wqkv": weight(rows, h, tensor_seed(s, SLOT_WQKV), dtype),
        "Wo": weight(h, nh * d, tensor_seed(s, SLOT_WO), dtype),
    }
    if with_bias:
        out["bqkv"] = bias(rows, tensor_seed(s, SLOT_BQKV), dtype)
        out["bo"] = bias(h, tensor_seed(s, SLOT_BO), dtype)
    return out


def as_numpy_f64(t: torch.Tensor):
    """Exact widening of stored values (bf16 or fp32) to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
