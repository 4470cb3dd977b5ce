"""Benchmark of one GPU's tensor-parallel shard path on MI355X.

A step is one pass of the whole shard path of a Llama-70B-shaped layer at TP = 8
and 4096 prefill tokens, every shard looped on this GPU:
  for each shard r: QKV_r = X Wqkv_r^T + bqkv_r                 (column, head split)
                    P_r   = Q_r Wo_r^T                          (row partial, A := Q)
  Y1 = sum_r P_r + bo                                           (combine: sum)
  for each shard r: H_r = silu(Y1 Wg_r^T + bg_r) * (Y1 Wu_r^T + bu_r)   (column pair)
                    P_r = H_r Wd_r^T                            (row partial)
  Y  = sum_r P_r + bd                                           (combine: sum)
  QKV = concat_r QKV_r (Q | K | V segments), H = concat_r H_r   (combine: concat)
Taking the shards (index arithmetic and copies) happens once at load, untimed.

Prints one JSON line. Also measured in the same run: per-kernel times of the
layer, the decode shards (M <= 64, weights rotated through > 1 GiB of copies so
the 256 MB Infinity Cache cannot serve them), and the fp64 oracle on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the decode sections and print their JSON (for a kernel trace)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time")
    ap.add_argument("--traffic-copy-mib", type=int, default=0,
                    help="first run one plain contiguous copy of this many MiB (counter calibration)")
    ap.add_argument("--traffic-dma-check", action="store_true",
                    help="then one LDS-DMA GEMM whose every weight byte is read once (256 tokens x 65536 x 1024: "
                         "128 MiB of weights read, 32 MiB written), to check the calibration on DMA loads")
    ap.add_argument("--decode-iters", type=int, default=110, help="launches per decode measurement")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def reserve_for(fn):
    """Size the library's work space for the current stream with a dry run of fn (which
    validates and plans its calls but enqueues nothing), then reserve it. Setup only: the
    timed calls themselves never allocate."""
    import tensor_transformer_linear_col_amd as tp
    with tp.tp_plan() as need:
        fn()
    if need.partial_bytes or need.n_counters:
        tp.tp_workspace_reserve(need.partial_bytes, need.n_counters)
    return need


# ----------------------------------------------------------------------------------------
# The layer
# ----------------------------------------------------------------------------------------

class Layer:
    def __init__(self, shape):
        import torch
        import tensor_transformer_linear_col_amd as tp
        import tp_inputs as I
        self.tp, self.torch = tp, torch
        BF = torch.bfloat16
        s = shape
        self.M = M = s.tokens[0]
        self.h, self.inter, self.p = s.hidden, s.intermediate, s.tp
        self.nh, self.nkv, self.d = s.n_heads, s.n_kv_heads, s.head_dim
        p, h, inter = self.p, self.h, self.inter
        self.nq = (self.nh // p + 2 * self.nkv // p) * self.d
        self.ka = self.nh // p * self.d
        self.i = inter // p
        t0 = time.time()
        aw = I.attn_weights(s, with_bias=True)
        fw = I.ffn_weights(s, with_bias=True)
        x = I.activations(M, h, I.activation_seed(s.seed, M))
        log(f"inputs drawn in {time.time() - t0:.1f}s")
        dev = lambda t: t.contiguous().cuda()
        self.X = dev(x)
        self.bo, self.bd = dev(aw["bo"]), dev(fw["bd"])
        self.shards = []
        full = {k: dev(v) for k, v in {**aw, **fw}.items()}
        for r in range(p):
            sh = {}
            sh["Wqkv"] = torch.empty(self.nq, h, dtype=BF, device="cuda")
            sh["bqkv"] = torch.empty(self.nq, dtype=BF, device="cuda")
            tp.tp_shard_qkv(full["Wqkv"], h, self.nh, self.nkv, self.d, p, r, sh["Wqkv"])
            tp.tp_shard_qkv(full["bqkv"], 1, self.nh, self.nkv, self.d, p, r, sh["bqkv"])
            sh["Wo"] = torch.empty(h, self.ka, dtype=BF, device="cuda")
            tp.tp_shard_weight(full["Wo"], h, self.nh * self.d, p, r, 1, sh["Wo"])
            for nm in ("Wg", "Wu"):
                sh[nm] = torch.empty(self.i, h, dtype=BF, device="cuda")
                tp.tp_shard_weight(full[nm], inter, h, p, r, 0, sh[nm])
            for nm in ("bg", "bu"):
                sh[nm] = torch.empty(self.i, dtype=BF, device="cuda")
                tp.tp_shard_weight(full[nm], inter, 1, p, r, 0, sh[nm])
            sh["Wd"] = torch.empty(h, self.i, dtype=BF, device="cuda")
            tp.tp_shard_weight(full["Wd"], h, inter, p, r, 1, sh["Wd"])
            sh["QKV"] = torch.empty(M, self.nq, dtype=BF, device="cuda")
            sh["Po"] = torch.empty(M, h, dtype=BF, device="cuda")
            sh["H"] = torch.empty(M, self.i, dtype=BF, device="cuda")
            sh["Pd"] = torch.empty(M, h, dtype=BF, device="cuda")
            self.shards.append(sh)
        del full
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        self.Y1 = torch.empty(M, h, dtype=BF, device="cuda")
        self.Y = torch.empty(M, h, dtype=BF, device="cuda")
        self.QKVc = torch.empty(M, (self.nh + 2 * self.nkv) * self.d, dtype=BF, device="cuda")
        self.A = torch.empty(M, self.nh * self.d // self.p, dtype=BF, device="cuda")  # one shard's attention output
        self.Hc = torch.empty(M, inter, dtype=BF, device="cuda")
        self.seg = [self.nh // p * self.d, self.nkv // p * self.d, self.nkv // p * self.d]
        # algorithmic work per step (2 M N K per product)
        self.flops = {
            "qkv": 2.0 * M * self.nq * h * p,
            "o": 2.0 * M * h * self.ka * p,
            "gateup": 2.0 * 2 * M * self.i * h * p,
            "down": 2.0 * M * h * self.i * p,
        }
        self.total_flops = sum(self.flops.values())
        # The two concats only check the split; they run on a second stream (default
        # priority) and overlap the GEMMs that follow their inputs.
        self.side = torch.cuda.Stream()
        need = reserve_for(lambda: (self.step(), self.step(core=True)))
        log(f"work space: {need.partial_bytes / 2**20:.1f} MiB of partials, {need.n_counters} counters")

    def step(self, ev=None, core=False, only=None):
        """One pass of the shard path. ev: optional dict name -> list of (start, end) events,
        recorded around the launches named in `only` (all when None). core: run the head-local
        attention core between QKV and O instead of A := Q. The concats run on the side stream
        (each after its inputs are written, the step ending when both are done), except when
        every launch is timed, where they stay on the main stream to be timed too."""
        tp, torch = self.tp, self.torch
        M, h, p = self.M, self.h, self.p
        overlap = not (ev is not None and only is None)
        main = torch.cuda.current_stream()

        def on_side(fn):
            done = torch.cuda.Event()
            done.record(main)
            self.side.wait_event(done)
            with torch.cuda.stream(self.side):
                fn()

        def timed(name, fn):
            if ev is None or (only is not None and name not in only):
                fn()
                return
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev.setdefault(name, []).append((a, b))

        for sh in self.shards:
            timed("qkv", lambda: tp.tp_attn_proj_shard(self.X, sh["Wqkv"], sh["bqkv"], sh["QKV"], None, None, None,
                                                      M, h, self.nh, self.nkv, self.d, p))
            if core:
                timed("core", lambda: tp.tp_attn_core_shard(sh["QKV"], self.A, M, self.nh, self.nkv, self.d, p, True))
                timed("o", lambda: tp.tp_linear_row_partial(self.A, self.nh * self.d // p, sh["Wo"], sh["Po"], M,
                                                            self.nh * self.d, h, p))
                continue
            # A := Q: the shard's Q heads are the first ka columns of QKV_r (row stride nq)
            timed("o", lambda: tp.tp_linear_row_partial(sh["QKV"], self.nq, sh["Wo"], sh["Po"], M,
                                                        self.nh * self.d, h, p))
        concat_qkv = lambda: tp.tp_combine_concat([sh["QKV"] for sh in self.shards], self.seg, self.QKVc, M)
        concat_h = lambda: tp.tp_combine_concat([sh["H"] for sh in self.shards], [self.i], self.Hc, M)
        if overlap:
            on_side(concat_qkv)
        timed("sum", lambda: tp.tp_combine_sum([sh["Po"] for sh in self.shards], self.bo, self.Y1, M, h))
        for r, sh in enumerate(self.shards):
            timed("gateup", lambda: tp.tp_mlp_shard(self.Y1, sh["Wg"], sh["Wu"], sh["bg"], sh["bu"], None,
                                                    sh["H"], None, M, h, self.inter, p))
            if overlap and r == p - 1:
                on_side(concat_h)
            timed("down", lambda: tp.tp_linear_row_partial(sh["H"], self.i, sh["Wd"], sh["Pd"], M, self.inter,
                                                           h, p))
        timed("sum", lambda: tp.tp_combine_sum([sh["Pd"] for sh in self.shards], self.bd, self.Y, M, h))
        if overlap:
            main.wait_stream(self.side)
        else:
            timed("concat_qkv", concat_qkv)
            timed("concat_h", concat_h)


def attention_bench(layer, reps=20):
    """The head-local attention core on each of the layer's 8 shards (its own QKV_r from the
    timed step: 8 query heads and 1 KV head of 128, causal over the 4096 tokens). Not part of
    the layer step above, whose attention stand-in is A := Q. Work per shard: 2 products of
    2 * d flops per (query, allowed key) pair and head: 4 * d * hq * M(M+1)/2. Also the whole
    layer step with the core in place of the stand-in (QKV -> core -> O per shard), whose
    work adds the 8 shards' attention flops to the layer's GEMM flops."""
    import torch
    tp = layer.tp
    M, p, d = layer.M, layer.p, layer.d
    hq = layer.nh // p
    A = torch.empty(M, hq * d, dtype=torch.bfloat16, device="cuda")
    run = lambda: [tp.tp_attn_core_shard(sh["QKV"], A, M, layer.nh, layer.nkv, d, p, True) for sh in layer.shards]
    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (reps * p)
    flops = 4.0 * d * hq * M * (M + 1) / 2
    tf = flops / (us * 1e-6) / 1e12
    log(f"attention core: {us:.1f} us per shard, {tf:.1f} TFLOP/s")

    layer.step(core=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        layer.step(core=True)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    lflops = layer.total_flops + p * flops
    ltf = lflops / (ms * 1e-3) / 1e12
    log(f"layer step with the attention core: {ms:.3f} ms, {ltf:.1f} TFLOP/s")
    return {"kernel": "attn_kernel (causal GQA, 8 query heads / 1 KV head of 128, 4096 tokens)",
            "us_per_shard": round(us, 1), "TFLOP_s": round(tf, 1), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
            "layer_step_with_core": {"ms_per_step": round(ms, 4), "GFLOP": round(lflops / 1e9, 1),
                                     "TFLOP_s": round(ltf, 1)}}


def attention_decode_bench(reps=50):
    """One decode step of the attention core over a KV cache on the 70B TP=8 shard (8 query
    heads, 1 KV head of 128): new tokens M appended at position T, attention over T + M keys.
    Bytes: the K and V cache rows read once, (T + M) * 2 * 128 * 2."""
    import torch
    import tensor_transformer_linear_col_amd as tp
    nh, nkv, d, p = 64, 8, 128, 8
    hq, hk = nh // p, nkv // p
    g = torch.Generator().manual_seed(7)
    out = []
    for T in (4096, 32768):
        Kc = torch.randn(T + 64, hk * d, generator=g).to(torch.bfloat16).cuda()
        Vc = torch.randn(T + 64, hk * d, generator=g).to(torch.bfloat16).cuda()
        for M in (1, 16):
            Q = torch.randn(M, (hq + 2 * hk) * d, generator=g).to(torch.bfloat16).cuda()
            A = torch.empty(M, hq * d, dtype=torch.bfloat16, device="cuda")
            reserve_for(lambda: tp.tp_attn_decode_shard(Q, Kc, Vc, T, A, M, nh, nkv, d, p))
            tp.tp_attn_decode_shard(Q, Kc, Vc, T, A, M, nh, nkv, d, p)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                tp.tp_attn_decode_shard(Q, Kc, Vc, T, A, M, nh, nkv, d, p)
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / reps
            gbs = (T + M) * 2 * hk * d * 2 / (us * 1e-6) / 1e9
            log(f"attention decode T={T} M={M}: {us:.1f} us, {gbs:.0f} GB/s")
            out.append({"cache_len": T, "M": M, "us": round(us, 2), "GB_s": round(gbs, 1)})
    return {"kernels": "append_kv_kernel + attn_kernel (packed query heads, cut keys) + attn_merge_kernel", "steps": out}


def kernel_ms(ev):
    out = {}
    for name, pairs in ev.items():
        ms = [a.elapsed_time(b) for a, b in pairs]
        out[name] = sum(ms) / len(ms)
    return out


# ----------------------------------------------------------------------------------------
# Decode shards (M <= 64): HBM-bound, weights rotated through > 1 GiB of copies
# ----------------------------------------------------------------------------------------

def hold_gpu(seconds):
    import torch
    try:
        torch.cuda._sleep(int(seconds * 2.4e9))
    except Exception:
        pass


def decode_bench(iters=100):
    import torch
    import tensor_transformer_linear_col_amd as tp
    import tp_inputs as I
    BF = torch.bfloat16
    results = []
    for shape in (I.LLAMA7B_FFN_TP2, I.LLAMA70B_FFN_TP4):
        h, inter, p = shape.hidden, shape.intermediate, shape.tp
        i = inter // p
        wt = I.ffn_weights(shape, with_bias=False)
        shard_bytes = 3 * i * h * 2
        copies = max(1, -(-(1 << 30) // shard_bytes) + 1)
        sets = []
        base = [(wt["Wg"][r * i:(r + 1) * i].contiguous().cuda(), wt["Wu"][r * i:(r + 1) * i].contiguous().cuda(),
                 wt["Wd"][:, r * i:(r + 1) * i].contiguous().cuda()) for r in range(p)]
        for c in range(copies):
            sets.append(base[c % p] if c < p else tuple(t.clone() for t in base[c % p]))
        del wt
        for M in shape.tokens:
            x = I.activations(M, h, I.activation_seed(shape.seed, M)).cuda()
            H = torch.empty(M, i, dtype=BF, device="cuda")
            P = torch.empty(M, h, dtype=BF, device="cuda")
            reserve_for(lambda: (tp.tp_mlp_shard(x, *sets[0][:2], None, None, None, H, None, M, h, inter, p),
                                 tp.tp_linear_row_partial(H, i, sets[0][2], P, M, inter, h, p)))
            for c in range(len(sets)):  # warm
                Wg, Wu, Wd = sets[c]
                tp.tp_mlp_shard(x, Wg, Wu, None, None, None, H, None, M, h, inter, p)
            torch.cuda.synchronize()
            # Keep the GPU busy (a bounded spin) while the timed launches are queued, so the
            # events time the kernels and not the host's launch rate.
            hold_gpu(5e-3)
            ev_g, ev_d = [], []
            for it in range(iters):
                Wg, Wu, Wd = sets[it % len(sets)]
                a, b, c2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                a.record()
                tp.tp_mlp_shard(x, Wg, Wu, None, None, None, H, None, M, h, inter, p)
                b.record()
                tp.tp_linear_row_partial(H, i, Wd, P, M, inter, h, p)
                c2.record()
                ev_g.append((a, b))
                ev_d.append((b, c2))
            torch.cuda.synchronize()
            gu = sorted(a.elapsed_time(b) for a, b in ev_g)[len(ev_g) // 2]
            dn = sorted(a.elapsed_time(b) for a, b in ev_d)[len(ev_d) // 2]
            # The same launches back to back (one event pair around all of them, weights still
            # rotated): the per-launch events above also time each launch's dispatch and the
            # event records themselves, which a stream of layer kernels overlaps.
            stream_ms = {}
            for op in ("gateup_swiglu", "down_partial"):
                hold_gpu(5e-3)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for it in range(iters):
                    Wg, Wu, Wd = sets[it % len(sets)]
                    if op == "gateup_swiglu":
                        tp.tp_mlp_shard(x, Wg, Wu, None, None, None, H, None, M, h, inter, p)
                    else:
                        tp.tp_linear_row_partial(H, i, Wd, P, M, inter, h, p)
                b.record()
                torch.cuda.synchronize()
                stream_ms[op] = a.elapsed_time(b) / iters
            gu_bytes = 2 * i * h * 2 + M * h * 2 + M * i * 2
            dn_bytes = h * i * 2 + M * i * 2 + M * h * 2
            for op, ms, by, fl in (("gateup_swiglu", gu, gu_bytes, 2.0 * 2 * M * i * h),
                                   ("down_partial", dn, dn_bytes, 2.0 * M * h * i)):
                gbs = by / (ms * 1e-3) / 1e9
                sgbs = by / (stream_ms[op] * 1e-3) / 1e9
                results.append({"workload": shape.name, "M": M, "op": op, "us": round(ms * 1e3, 2),
                                "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 3),
                                "TFLOP_s": round(fl / (ms * 1e-3) / 1e12, 2),
                                "us_back_to_back": round(stream_ms[op] * 1e3, 2),
                                "hbm_frac_back_to_back": round(sgbs / HBM_PEAK_GBS, 3)})
            log(f"decode {shape.name} M={M}: gate/up {gu*1e3:.1f} us, down {dn*1e3:.1f} us "
                f"(back to back: {stream_ms['gateup_swiglu']*1e3:.1f} / {stream_ms['down_partial']*1e3:.1f} us)")
        del sets, base
        torch.cuda.empty_cache()

    # The pages' own FFN (GELU between the column and the row layer), batch 4, TP = 2.
    shape = I.PAGES_FFN_GELU_TP2
    h, inter, p = shape.hidden, shape.intermediate, shape.tp
    i = inter // p
    wt = I.gelu_ffn_weights(shape, with_bias=True)
    shard_bytes = 2 * i * h * 2
    copies = max(1, -(-(1 << 30) // shard_bytes) + 1)
    base = [(wt["W1"][r * i:(r + 1) * i].contiguous().cuda(), wt["b1"][r * i:(r + 1) * i].contiguous().cuda(),
             wt["W2"][:, r * i:(r + 1) * i].contiguous().cuda()) for r in range(p)]
    sets = [base[c % p] if c < p else tuple(t.clone() for t in base[c % p]) for c in range(copies)]
    del wt
    for M in shape.tokens:
        x = I.activations(M, h, I.activation_seed(shape.seed, M)).cuda()
        H = torch.empty(M, i, dtype=BF, device="cuda")
        P = torch.empty(M, h, dtype=BF, device="cuda")
        reserve_for(lambda: (tp.tp_ffn_gelu_shard(x, sets[0][0], sets[0][1], None, H, None, M, h, inter, p),
                             tp.tp_linear_row_partial(H, i, sets[0][2], P, M, inter, h, p)))
        for c in range(len(sets)):  # warm
            W1, b1, W2 = sets[c]
            tp.tp_ffn_gelu_shard(x, W1, b1, None, H, None, M, h, inter, p)
        torch.cuda.synchronize()
        hold_gpu(5e-3)
        ev_c, ev_r = [], []
        for it in range(iters):
            W1, b1, W2 = sets[it % len(sets)]
            a, b, c2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            a.record()
            tp.tp_ffn_gelu_shard(x, W1, b1, None, H, None, M, h, inter, p)
            b.record()
            tp.tp_linear_row_partial(H, i, W2, P, M, inter, h, p)
            c2.record()
            ev_c.append((a, b))
            ev_r.append((b, c2))
        torch.cuda.synchronize()
        cu = sorted(a.elapsed_time(b) for a, b in ev_c)[len(ev_c) // 2]
        rw = sorted(a.elapsed_time(b) for a, b in ev_r)[len(ev_r) // 2]
        cu_bytes = i * h * 2 + i * 2 + M * h * 2 + M * i * 2
        rw_bytes = h * i * 2 + M * i * 2 + M * h * 2
        for op, ms, by, fl in (("col_gelu", cu, cu_bytes, 2.0 * M * i * h), ("row_partial", rw, rw_bytes, 2.0 * M * h * i)):
            gbs = by / (ms * 1e-3) / 1e9
            results.append({"workload": shape.name, "M": M, "op": op, "us": round(ms * 1e3, 2),
                            "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 3),
                            "TFLOP_s": round(fl / (ms * 1e-3) / 1e12, 2)})
        log(f"decode {shape.name} M={M}: column+gelu {cu*1e3:.1f} us, row {rw*1e3:.1f} us")
    del sets, base
    torch.cuda.empty_cache()
    results += split_variants_bench(iters)
    return results


def _median_launch_us(fn, n_sets, iters):
    import torch
    hold_gpu(5e-3)
    evs = []
    for it in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(it % n_sets)
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in evs)[len(evs) // 2] * 1e3


def stream_reference_bench(iters=60):
    """A plain device copy (torch's copy kernel, one read and one write of every byte) at the
    byte sizes of the decode shards, sources rotated through > 1 GiB: how close a kernel with
    no arithmetic comes to the HBM rate at each size, i.e. the fixed cost of launching,
    ramping up and draining a short stream on this chip."""
    import torch
    out = []
    for mb in (16.8, 21.0, 45.1, 90.2, 117.4, 234.9):
        n = int(mb * 1e6) // 2 // 8 * 8
        copies = max(2, -(-(1 << 30) // (2 * n)) + 1)
        srcs = [torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0) for _ in range(copies)]
        dst = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        fn = lambda c: dst.copy_(srcs[c])
        for c in range(copies):
            fn(c)
        torch.cuda.synchronize()
        us = _back_to_back_us(fn, copies, iters)
        gbs = 2 * n * 2 / us / 1e3
        out.append({"MB_read": round(2 * n / 1e6, 1), "us_back_to_back": round(us, 2), "GB_s_read_plus_write": round(gbs, 1),
                    "hbm_frac": round(gbs / HBM_PEAK_GBS, 3)})
        del srcs, dst
    torch.cuda.empty_cache()
    log("plain copy reference: " + ", ".join(f"{r['MB_read']} MB {r['hbm_frac']}" for r in out))
    return {"kernel": "torch copy_ (read + write)", "sizes": out}


def _back_to_back_us(fn, n_sets, iters):
    """The same launches back to back between one pair of events (the rate of a stream of
    such kernels), weights still rotated."""
    import torch
    hold_gpu(5e-3)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for it in range(iters):
        fn(it % n_sets)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / iters


def attnproj_bench(iters=100):
    """The 70B attention-projection shard at TP = 8 (64 query / 8 KV heads of 128, hidden
    8192): the QKV column product 8192 -> 1280 (8 Q heads, 1 K, 1 V) and the O row partial
    1024 -> 8192. At one token (decode, HBM-bound) the weights rotate through > 1 GiB of
    copies so the 256 MB Infinity Cache cannot serve them; at 2048 tokens (prefill,
    MFMA-bound) the 8 shards' weights are taken in turn. Algorithmic bytes: weights + X +
    output; flops: 2 M N K."""
    import torch
    import tensor_transformer_linear_col_amd as tp
    import tp_inputs as I
    BF = torch.bfloat16
    shape = I.LLAMA70B_ATTN_TP8
    h, nh, nkv, d, p = shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.tp
    nq, ka = (nh // p + 2 * nkv // p) * d, nh // p * d
    wt = I.attn_weights(shape, with_bias=False)
    Wqkv, Wo = wt["Wqkv"].cuda(), wt["Wo"].cuda()
    base = []
    for r in range(p):
        wq = torch.empty(nq, h, dtype=BF, device="cuda")
        wo = torch.empty(h, ka, dtype=BF, device="cuda")
        tp.tp_shard_qkv(Wqkv, h, nh, nkv, d, p, r, wq)
        tp.tp_shard_weight(Wo, h, nh * d, p, r, 1, wo)
        base.append((wq, wo))
    del Wqkv, Wo, wt
    shard_bytes = (nq * h + h * ka) * 2
    copies = max(p, -(-(1 << 30) // shard_bytes) + 1)
    sets = base + [tuple(t.clone() for t in base[c % p]) for c in range(p, copies)]
    out = []
    for M in shape.tokens:
        x = I.activations(M, h, I.activation_seed(shape.seed, M)).cuda()
        a = I.activations(M, ka, I.activation_seed(shape.seed, M, slot=1)).cuda()
        QKV = torch.empty(M, nq, dtype=BF, device="cuda")
        P = torch.empty(M, h, dtype=BF, device="cuda")
        qkv_fn = lambda c: tp.tp_attn_proj_shard(x, sets[c][0], None, QKV, None, None, None, M, h, nh, nkv, d, p)
        o_fn = lambda c: tp.tp_attn_proj_shard(None, None, None, None, a, sets[c][1], P, M, h, nh, nkv, d, p)
        reserve_for(lambda: (qkv_fn(0), o_fn(0)))
        n_sets = len(sets) if M <= 64 else p
        for c in range(n_sets):  # warm
            qkv_fn(c)
            o_fn(c)
        torch.cuda.synchronize()
        n_it = iters if M <= 64 else max(16, iters // 4)
        for op, fn, by, fl in (("qkv_col", qkv_fn, nq * h * 2 + M * h * 2 + M * nq * 2, 2.0 * M * nq * h),
                               ("o_row_partial", o_fn, h * ka * 2 + M * ka * 2 + M * h * 2, 2.0 * M * h * ka)):
            us = _median_launch_us(fn, n_sets, n_it)
            us_b2b = _back_to_back_us(fn, n_sets, n_it)
            rec = {"workload": shape.name, "M": M, "op": op, "us": round(us, 2), "us_back_to_back": round(us_b2b, 2),
                   "GB_s": round(by / us / 1e3, 1), "TFLOP_s": round(fl / us / 1e6, 2)}
            if M <= 64:
                # at one token the QKV shard's 80 row groups of 16 take the GEMV kernel (fewer than CUs)
                rec["kernel"] = "gemv_kernel" if op == "qkv_col" else "skinny_kernel"
                rec["hbm_frac"] = round(by / us / 1e3 / HBM_PEAK_GBS, 3)
                rec["hbm_frac_back_to_back"] = round(by / us_b2b / 1e3 / HBM_PEAK_GBS, 3)
            else:
                # 2048 tokens: QKV as 128 tiles of 160 x 128 in 2 K ranges + their reduce; O on 256 x 256 tiles
                rec["kernel"] = ("gemm_dtl16_kernel + splitk16_reduce_kernel" if op == "qkv_col" else "gemm_dtl_kernel")
                rec["bf16_frac"] = round(fl / us / 1e6 / BF16_PEAK_TFLOPS, 4)
                rec["bf16_frac_back_to_back"] = round(fl / us_b2b / 1e6 / BF16_PEAK_TFLOPS, 4)
            out.append(rec)
            log(f"attention projection {shape.name} M={M} {op}: {us:.1f} us per launch, {us_b2b:.1f} us back to back")
    del sets, base
    torch.cuda.empty_cache()
    return out


def split_variants_bench(iters=100):
    """Decode shards of the two split variants: an uneven column split (the 7B FFN's 11008
    gate rows over 3 shards, 3672 + 3672 + 3664, which the listing's divisibility assert would
    reject) and a QKV shard with KV-head replication (70B attention at TP = 16: 4 Q heads and
    one of the 8 KV heads per shard). Weights rotated through > 1 GiB; M = 1."""
    import torch
    import tensor_transformer_linear_col_amd as tp
    import tp_inputs as I
    BF = torch.bfloat16
    out = []
    # uneven column split, shard 0 (the widest)
    h, width = 4096, 3672
    w = I.weight(width, h, seed=901).cuda()
    copies = 1 + (1 << 30) // (width * h * 2)
    sets = [w] + [w.clone() for _ in range(copies - 1)]
    x = I.activations(1, h, seed=902).cuda()
    y = torch.empty(1, width, dtype=BF, device="cuda")
    fn = lambda c: tp.tp_linear_col(x, sets[c], None, y, 1, h, width, 1)
    reserve_for(lambda: fn(0))
    for c in range(len(sets)):
        fn(c)
    torch.cuda.synchronize()
    us = _median_launch_us(fn, len(sets), iters)
    by = width * h * 2 + h * 2 + width * 2
    out.append({"workload": "llama7b-ffn-uneven-tp3 (shard 0 of 3672/3672/3664)", "M": 1, "op": "col",
                "us": round(us, 2), "GB_s": round(by / us / 1e3, 1), "hbm_frac": round(by / us / 1e3 / HBM_PEAK_GBS, 3),
                "TFLOP_s": round(2.0 * width * h / us / 1e6, 3)})
    del sets, w
    # QKV shard with KV-head replication
    nh, nkv, d, hid, p = 64, 8, 128, 8192, 16
    nq = (nh // p + 2) * d
    wq = I.weight(nq, hid, seed=903).cuda()
    copies = 1 + (1 << 30) // (nq * hid * 2)
    sets = [wq] + [wq.clone() for _ in range(copies - 1)]
    x = I.activations(1, hid, seed=904).cuda()
    q = torch.empty(1, nq, dtype=BF, device="cuda")
    fn = lambda c: tp.tp_attn_proj_shard(x, sets[c], None, q, None, None, None, 1, hid, nh, nkv, d, p)
    reserve_for(lambda: fn(0))
    for c in range(len(sets)):
        fn(c)
    torch.cuda.synchronize()
    us = _median_launch_us(fn, len(sets), iters)
    by = nq * hid * 2 + hid * 2 + nq * 2
    out.append({"workload": "llama70b-qkv-tp16-kv-replicated", "M": 1, "op": "qkv",
                "us": round(us, 2), "GB_s": round(by / us / 1e3, 1), "hbm_frac": round(by / us / 1e3 / HBM_PEAK_GBS, 3),
                "TFLOP_s": round(2.0 * nq * hid / us / 1e6, 3)})
    del sets, wq
    torch.cuda.empty_cache()
    log(f"decode split variants: " + ", ".join(f"{r['workload']} {r['us']} us" for r in out))
    return out


# ----------------------------------------------------------------------------------------
# The fp64 oracle on the host, on a bounded sample of the same workload
# ----------------------------------------------------------------------------------------

def cpu_baseline(shape, target_s):
    import numpy as np
    import oracle as O
    import tp_inputs as I
    host_cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        threads = max([d.get("num_threads", 1) for d in blas] or [1])
        backend = ", ".join(sorted({f"{d.get('internal_api')} {d.get('version')}" for d in blas})) or "unknown"
    except Exception:
        threads, backend = host_cores, "unknown"
    aw = I.attn_weights(shape, with_bias=True)
    fw = I.ffn_weights(shape, with_bias=True)
    w = {k: I.as_numpy_f64(v) for k, v in {**aw, **fw}.items()}
    w.update(n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim)
    del aw, fw
    M = shape.tokens[0]
    x = I.as_numpy_f64(I.activations(M, shape.hidden, I.activation_seed(shape.seed, M)))
    flop_per_token = 2.0 * shape.hidden * ((shape.n_heads + 2 * shape.n_kv_heads) * shape.head_dim
                                           + shape.n_heads * shape.head_dim + 3 * shape.intermediate)
    S = 16
    while True:
        t0 = time.perf_counter()
        O.layer_unsharded(x[:S], w)
        dt = time.perf_counter() - t0
        if dt >= target_s * 0.5 or S >= M:
            break
        S = int(min(M, max(2 * S, S * target_s / max(dt, 1e-3))))
    tflops = S * flop_per_token / dt / 1e12
    return {"value": round(tflops, 4), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "host_cores_available": host_cores, "blas_backend": backend, "blas_threads": int(threads),
            "sample": f"{S} of {M} tokens through the unsharded fp64 layer chain (numpy float64 BLAS), "
                      f"{dt:.1f} s"}


def traffic_for(kernel_src, name):
    """HBM bytes per launch from stored rocprofv3 counter runs, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's shard path; --gpus {args.gpus} is not supported "
              "(the cross-shard combine runs on one device here)", file=sys.stderr)
        sys.exit(2)
    import torch
    import tp_inputs as I
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.decode_only:
        print(json.dumps({"decode": decode_bench(args.decode_iters), "attention_projection": attnproj_bench(args.decode_iters),
                          "attention_decode": attention_decode_bench(),
                          "stream_reference": stream_reference_bench()}), flush=True)
        return
    if args.traffic_copy_mib > 0:
        # A plain copy of known size: reads and writes exactly n bytes each. Under
        # rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE it calibrates the counters.
        import tensor_transformer_linear_col_amd as tp
        cols = 8192
        rows = args.traffic_copy_mib * (1 << 20) // (2 * cols)
        src = torch.ones(rows, cols, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        tp.tp_shard_weight(src, rows, cols, 1, 0, 0, dst)
        torch.cuda.synchronize()
        del src, dst
        if args.traffic_dma_check:
            M, N, K = 256, 65536, 1024  # 256 tiles of 256 x 256 on the LDS-DMA kernel, one per CU
            x = torch.ones(M, K, dtype=torch.bfloat16, device="cuda")
            w = torch.ones(N, K, dtype=torch.bfloat16, device="cuda")
            y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            tp.tp_linear_col(x, w, None, y, M, K, N, 1)
            torch.cuda.synchronize()
            del x, w, y
    shape = I.LLAMA70B_LAYER_TP8
    layer = Layer(shape)

    for _ in range(args.warmup):
        layer.step()
    torch.cuda.synchronize()
    # The timed region: events only around the dominant kernel's launches (for its roofline);
    # an event pair around every launch would put 72 event commands between the step's kernels.
    ev = {}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer.step(ev, only=("gateup",))
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt / args.steps * 1e3
    gu_ms = kernel_ms(ev)["gateup"]  # ms per launch, inside the timed region
    # Every other launch's duration from a few more steps with events around every launch.
    ev_all = {}
    for _ in range(3):
        layer.step(ev_all)
    torch.cuda.synchronize()
    per = kernel_ms(ev_all)
    per["gateup"] = gu_ms
    tflops = layer.total_flops / (ms_step * 1e-3) / 1e12
    log(f"layer step {ms_step:.3f} ms, {tflops:.1f} TFLOP/s; per launch (ms): "
        + ", ".join(f"{k} {v:.4f}" for k, v in per.items()))

    # dominant kernel: the fused gate/up + SwiGLU product (55% of the layer's flops)
    gu_flops = layer.flops["gateup"] / layer.p
    achieved = gu_flops / (gu_ms * 1e-3) / 1e12
    traffic = traffic_for(os.path.join(ROOT, "tensor_transformer_linear_col_amd", "csrc", "k_gemm.hip"),
                          "gemm_gateup_swiglu_llama70b_tp8_m4096")
    kernels = {}
    for name in ("qkv", "o", "gateup", "down"):
        fl = layer.flops[name] / layer.p
        kernels[name] = {"us_per_launch": round(per[name] * 1e3, 1),
                         "TFLOP_s": round(fl / (per[name] * 1e-3) / 1e12, 1)}
    M, h = layer.M, layer.h
    sum_bytes = (layer.p + 1) * M * h * 2 + h * 2
    kernels["combine_sum"] = {"us_per_launch": round(per["sum"] * 1e3, 1),
                              "GB_s": round(sum_bytes / (per["sum"] * 1e-3) / 1e9, 1)}
    for name, width in (("concat_qkv", layer.QKVc.shape[1]), ("concat_h", layer.Hc.shape[1])):
        by = 2 * M * width * 2  # every element read once and written once
        kernels[f"combine_{name}"] = {"us_per_launch": round(per[name] * 1e3, 1),
                                      "GB_s": round(by / (per[name] * 1e-3) / 1e9, 1)}

    attention = attention_bench(layer)
    decode = None if args.skip_decode else decode_bench(args.decode_iters)
    attention_decode = None if args.skip_decode else attention_decode_bench()
    attention_projection = None if args.skip_decode else attnproj_bench(args.decode_iters)
    stream_reference = None if args.skip_decode else stream_reference_bench()
    cpu = None if args.skip_cpu_baseline else cpu_baseline(shape, args.cpu_seconds)

    out = {
        "metric": "TP-shard GEMM TFLOP/s + HBM GB/s (decode M=1..64, prefill M=4096), 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights and biases, N(0,1) activations)",
        "config": {"workload": "llama70b-layer-prefill-tp8: all 8 shards of a 70B layer's QKV/O/gate/up/down "
                               "products at 4096 tokens looped on one GPU, with on-device sum and concat combines",
                   "tp_size": layer.p, "tokens": layer.M, "hidden": layer.h, "intermediate": layer.inter,
                   "n_heads": layer.nh, "n_kv_heads": layer.nkv, "head_dim": layer.d,
                   "flop_per_step": layer.total_flops},
        "roofline": {"kernel": "gemm_dtl_kernel gate/up + SwiGLU (one shard, 4096 x 3584 x 8192, x2)",
                     "bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": traffic},
        "kernels": kernels,
        "attention_core": attention,
        "decode": decode,
        "attention_projection": attention_projection,
        "attention_decode": attention_decode,
        "stream_reference": stream_reference,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
