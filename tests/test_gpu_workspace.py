"""The work-space contract on the GPU: a call whose split reduction needs more work space
than is reserved for its stream enqueues nothing; a dry run sizes the reservation; and
the layer step (prefill and decode sizes) replays under HIP graph capture, since no call
allocates, frees or synchronises."""
import pytest
import torch

import oracle as O
import tensor_transformer_linear_col_amd as tp
import tp_inputs as I
from gpu_util import BF16_TOL, dev, err, host64, log_case

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def test_unreserved_stream_refuses_and_enqueues_nothing():
    """The 70B QKV shard at 8 tokens cuts K across workgroups (partials + counters). On a
    stream with no reservation the call returns TP_ERR_WORKSPACE and its output is left
    untouched; after a reservation sized by a dry run it matches the null stream's result."""
    log_case("workspace refusal", "qkv tp8 M=8")
    M, h, nh, nkv, d, p = 8, 8192, 64, 8, 128, 8
    nq = (nh // p + 2 * nkv // p) * d
    X = dev(I.activations(M, h, 501))
    W = dev(I.weight(nq, h, 502))
    ref = torch.empty(M, nq, dtype=BF, device="cuda")
    tp.tp_attn_proj_shard(X, W, None, ref, None, None, None, M, h, nh, nkv, d, p)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Y = torch.full((M, nq), float("nan"), dtype=BF, device="cuda")
        torch.cuda.synchronize()
        with pytest.raises(tp.TPError) as e:
            tp.tp_attn_proj_shard(X, W, None, Y, None, None, None, M, h, nh, nkv, d, p)
        assert e.value.status == tp.TP_ERR_WORKSPACE
        torch.cuda.synchronize()
        assert torch.isnan(Y).all()
        with tp.tp_plan() as need:
            tp.tp_attn_proj_shard(X, W, None, Y, None, None, None, M, h, nh, nkv, d, p)
        assert need.partial_bytes > 0 and need.n_counters >= nq // 32
        torch.cuda.synchronize()
        assert torch.isnan(Y).all()  # the dry run enqueued nothing
        tp.tp_workspace_reserve(need.partial_bytes, need.n_counters)
        assert tp.tp_workspace_reserved() >= (need.partial_bytes, need.n_counters)
        tp.tp_attn_proj_shard(X, W, None, Y, None, None, None, M, h, nh, nkv, d, p)
    torch.cuda.synchronize()
    assert torch.equal(Y, ref)


class SmallLayer:
    """A layer step with every shard looped: QKV (column, head split) -> A := Q -> O partials
    -> sum + bo -> gate/up + SwiGLU -> down partials -> sum + bd."""

    def __init__(self, M, hidden, intermediate, n_heads, n_kv_heads, head_dim, p):
        shape = I.LayerShape("graph-test", hidden=hidden, intermediate=intermediate, n_heads=n_heads,
                             n_kv_heads=n_kv_heads, head_dim=head_dim, tp=p, tokens=(M,), seed=41)
        self.shape, self.M = shape, M
        self.aw = I.attn_weights(shape, with_bias=True)
        self.fw = I.ffn_weights(shape, with_bias=True)
        self.x = I.activations(M, shape.hidden, 4100 + M)
        h, p, nh, nkv, d, inter = shape.hidden, shape.tp, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.intermediate
        self.nq, self.ka, self.i = (nh // p + 2 * nkv // p) * d, nh // p * d, inter // p
        self.X = dev(self.x)
        full = {k: dev(v) for k, v in {**self.aw, **self.fw}.items()}
        self.sh = []
        for r in range(p):
            s = {"Wqkv": torch.empty(self.nq, h, dtype=BF, device="cuda"),
                 "bqkv": torch.empty(self.nq, dtype=BF, device="cuda"),
                 "Wo": torch.empty(h, self.ka, dtype=BF, device="cuda"),
                 "Wd": torch.empty(h, self.i, dtype=BF, device="cuda")}
            tp.tp_shard_qkv(full["Wqkv"], h, nh, nkv, d, p, r, s["Wqkv"])
            tp.tp_shard_qkv(full["bqkv"], 1, nh, nkv, d, p, r, s["bqkv"])
            tp.tp_shard_weight(full["Wo"], h, nh * d, p, r, 1, s["Wo"])
            for nm in ("Wg", "Wu"):
                s[nm] = torch.empty(self.i, h, dtype=BF, device="cuda")
                tp.tp_shard_weight(full[nm], inter, h, p, r, 0, s[nm])
            for nm in ("bg", "bu"):
                s[nm] = torch.empty(self.i, dtype=BF, device="cuda")
                tp.tp_shard_weight(full[nm], inter, 1, p, r, 0, s[nm])
            tp.tp_shard_weight(full["Wd"], h, inter, p, r, 1, s["Wd"])
            s["QKV"] = torch.empty(M, self.nq, dtype=BF, device="cuda")
            s["Po"] = torch.empty(M, h, dtype=BF, device="cuda")
            s["H"] = torch.empty(M, self.i, dtype=BF, device="cuda")
            s["Pd"] = torch.empty(M, h, dtype=BF, device="cuda")
            self.sh.append(s)
        self.bo, self.bd = full["bo"], full["bd"]
        self.Y1 = torch.empty(M, h, dtype=BF, device="cuda")
        self.Y = torch.empty(M, h, dtype=BF, device="cuda")
        torch.cuda.synchronize()

    def step(self):
        sh, M = self.shape, self.M
        h, p, nh, nkv, d, inter = sh.hidden, sh.tp, sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.intermediate
        for s in self.sh:
            tp.tp_attn_proj_shard(self.X, s["Wqkv"], s["bqkv"], s["QKV"], None, None, None, M, h, nh, nkv, d, p)
            tp.tp_linear_row_partial(s["QKV"], self.nq, s["Wo"], s["Po"], M, nh * d, h, p)
        tp.tp_combine_sum([s["Po"] for s in self.sh], self.bo, self.Y1, M, h)
        for s in self.sh:
            tp.tp_mlp_shard(self.Y1, s["Wg"], s["Wu"], s["bg"], s["bu"], s["Wd"], s["H"], s["Pd"], M, h, inter, p)
        tp.tp_combine_sum([s["Pd"] for s in self.sh], self.bd, self.Y, M, h)

    def reference(self):
        w = {k: host64(v) for k, v in {**self.aw, **self.fw}.items()}
        w.update(n_heads=self.shape.n_heads, n_kv_heads=self.shape.n_kv_heads, head_dim=self.shape.head_dim)
        return O.layer_unsharded(host64(self.x), w)


# Decode: 6 tokens, hidden 1024, 16 / 4 heads of 64, intermediate 2816 at TP = 4 (the QKV and
# gate/up products cut K across workgroups: partial tiles and arrival counters).
# Decode at 64 tokens: hidden 4096, 32 / 8 heads of 128, intermediate 11008 at TP = 2 (every
# product on LDS-staged 64-token tiles whose K ranges meet in a reduce pass).
# Prefill: 2048 tokens, the 70B attention shapes at TP = 8 with intermediate 4096 (the QKV
# and gate/up products run split-K with a reduce pass).
GRAPH_LAYERS = {"decode": (6, 1024, 2816, 16, 4, 64, 4), "decode64": (64, 4096, 11008, 32, 8, 128, 2),
                "prefill": (2048, 8192, 4096, 64, 8, 128, 8)}


@pytest.mark.parametrize("kind", list(GRAPH_LAYERS))
def test_layer_step_replays_under_graph_capture(kind):
    log_case("graph capture layer step", kind, GRAPH_LAYERS[kind])
    L = SmallLayer(*GRAPH_LAYERS[kind])
    with tp.tp_plan() as need:
        L.step()
    assert need.partial_bytes > 0  # every size exercises a split reduction
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        tp.tp_workspace_reserve(need.partial_bytes, need.n_counters)
        L.step()  # eager on the capture stream
    torch.cuda.synchronize()
    eager_y, eager_y1 = L.Y.clone(), L.Y1.clone()
    assert err(eager_y.cpu(), L.reference()) <= BF16_TOL
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        L.step()
    torch.cuda.synchronize()
    for rep in range(4):
        L.Y.fill_(float("nan"))
        L.Y1.fill_(float("nan"))
        L.step()  # eager work on the null stream between replays
        torch.cuda.synchronize()
        assert torch.equal(L.Y, eager_y)
        L.Y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(L.Y, eager_y), f"replay {rep}"
        assert torch.equal(L.Y1, eager_y1), f"replay {rep}"
    del g


@pytest.mark.parametrize("M,hq,hk,d", [(4096, 8, 1, 128), (2500, 16, 4, 64)])
def test_attention_core_replays_under_graph_capture(M, hq, hk, d):
    """The causal attention core where its key pieces merge through the work space (4096
    tokens, 8 heads: equal runs of the work order; 2500 tokens, head size 64: largest-first
    ranges), captured once and replayed with eager calls in between: every replay equals the
    eager result bitwise, so the arrival counters are back at zero after each run."""
    log_case("graph capture attention core", M, hq, hk, d)
    qkv = I.activations(M, (hq + 2 * hk) * d, 640 + M).cuda()
    A = torch.empty(M, hq * d, dtype=torch.bfloat16, device="cuda")
    with tp.tp_plan() as need:
        tp.tp_attn_core_shard(qkv, A, M, hq, hk, d, 1, True)
    assert need.partial_bytes > 0 and need.n_counters > 0
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        tp.tp_workspace_reserve(need.partial_bytes, need.n_counters)
        tp.tp_attn_core_shard(qkv, A, M, hq, hk, d, 1, True)
    torch.cuda.synchronize()
    eager = A.clone()
    assert err(eager.cpu(), O.attention_core_shard(host64(qkv.cpu()), hq, hk, d, True)) <= BF16_TOL
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        tp.tp_attn_core_shard(qkv, A, M, hq, hk, d, 1, True)
    torch.cuda.synchronize()
    for rep in range(4):
        A.fill_(float("nan"))
        tp.tp_attn_core_shard(qkv, A, M, hq, hk, d, 1, True)  # eager, null stream
        torch.cuda.synchronize()
        assert torch.equal(A, eager)
        A.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(A, eager), f"replay {rep}"
    del g
