#!/usr/bin/env python3
"""Benchmark of the fused decoder-layer ops on one MI355X.

A step is one pass of the four memory-bound ops over one synthetic batch of
32768 tokens (hidden 2048, 16 q / 8 kv heads of 128, intermediate 6144, bf16):
rmsnorm -> add_rmsnorm -> mrope (in place) -> swiglu, inputs resident in HBM.
`value` is the algorithmic bytes of a step over its time (GB/s).  Beside it
the same run times the decode-step op set (5 tokens x 28 layers of
add_rmsnorm -> mrope -> swiglu, and the 4-op layer with the post-attention
norm) replayed from one hipGraph, plus an empty-kernel graph with the same
node count as the launch floor.  `next_ops` times the ops built beside the
step (LayerNorm, M-RoPE + KV-cache append, softmax + top-k sampling, and
RMSNorm + Linear at the decode step's projection shapes and a prefill shape).

Every duration is taken with HIP events recorded on the stream the kernels
run on.  The oracle (the fp64 C reference) is timed on a bounded sample of the
same batch on the host for the CPU baseline.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
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

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_BF16_TFLOPS = 2500.0
METRIC = "achieved HBM GB/s (% of peak) per fused op; µs per decode-step op set"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_swiglu_prefill32k_bf16.json")
KERNEL_SOURCES = ["norm_rope_swiglu_amd/csrc/swiglu.hip", "norm_rope_swiglu_amd/csrc/device.hpp"]


def algorithmic_bytes(op, T, H, I, nq, nkv, D, s):
    """Bytes an op must move: each input read once, each output written once."""
    if op == "rmsnorm":
        return 2 * T * H * s + H * s
    if op == "add_rmsnorm":
        return 4 * T * H * s + H * s
    if op == "mrope":
        return 2 * (nq + nkv) * D * s * T + 12 * T
    if op == "swiglu":
        return 3 * T * I * s
    if op == "mrope_kv_append":   # q in place, k -> k cache, v -> v cache, 3 positions + seq + slot
        return 2 * (nq + 2 * nkv) * D * s * T + 20 * T
    if op == "layernorm":         # gamma and beta
        return 2 * T * H * s + 2 * H * s
    if op == "add_layernorm":
        return 4 * T * H * s + 2 * H * s
    raise ValueError(op)


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_counters(bytes_per_launch):
    """HBM bytes per swiglu launch from the committed rocprofv3 --pmc summary,
    or None when it is missing or the kernel changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, n_tokens, threads=None):
    """The oracle, untouched, on the first n_tokens of the batch: once on one
    host thread, and once with the tokens split into equal row shards, one
    per thread (the oracle's C functions keep no state, and ctypes drops the
    GIL around them).  The multi-thread run is the reported value."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle

    L = w.layer
    eps = float(np.float32(w.eps))
    gamma = L.gamma.cpu()

    def shard(a, b):
        sl = slice(a, b)
        return (L.x[sl].cpu(), L.residual[sl].cpu(), L.q[sl].cpu(), L.k[sl].cpu(),
                L.gate_up[sl].cpu(), w.pos[:, sl].cpu().contiguous())

    ops = (("rmsnorm", lambda s: oracle.rmsnorm(s[0], gamma, eps)),
           ("add_rmsnorm", lambda s: oracle.add_rmsnorm(s[0], s[1], gamma, eps)),
           ("mrope", lambda s: oracle.mrope(s[2], s[3], s[5], w.sections, w.theta)),
           ("swiglu", lambda s: oracle.swiglu(s[4])))
    byts = sum(algorithmic_bytes(op, n_tokens, w.hidden, w.inter, w.n_q, w.n_kv, w.head_dim, 2)
               for op in ("rmsnorm", "add_rmsnorm", "mrope", "swiglu"))

    def run(n_threads):
        cuts = [n_tokens * i // n_threads for i in range(n_threads + 1)]
        shards = [shard(cuts[i], cuts[i + 1]) for i in range(n_threads)]
        per_op_ms = {}
        with ThreadPoolExecutor(n_threads) as ex:
            t_all = time.perf_counter()
            for op, fn in ops:
                t0 = time.perf_counter()
                list(ex.map(fn, shards))
                per_op_ms[op] = round(1e3 * (time.perf_counter() - t0), 1)
            dt = time.perf_counter() - t_all
        return dt, per_op_ms

    if threads is None:
        # the host share this process may use (16 per GPU on the box), not every core in it
        threads = max(1, min(16, os.cpu_count() or 1))
    dt1, ms1 = run(1)
    dtn, msn = run(threads)
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(byts / dtn / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": round(dtn, 3), "per_op_ms": msn,
            "single_thread": {"value": round(byts / dt1 / 1e9, 3), "seconds": round(dt1, 2),
                              "per_op_ms": ms1},
            "host_cpu": cpu, "host_threads_available": os.cpu_count(),
            "sample": f"first {n_tokens} of {w.tokens} tokens of the step's batch, all four ops, "
                      f"fp64 C oracle on {threads} host threads (equal row shards), same "
                      "algorithmic-byte count; single_thread: the same on one thread"}


def op_sweep(dev, K=20, R=11, only=None):
    """Per-op launch duration and GB/s on every bandwidth-bound recipe: the
    2048-token prefill, the packed ragged batch and the 32768-token sweep at
    every width and dtype (head_dim 128, and M-RoPE again at head_dim 64).
    Each op's K launches are captured
    in one graph (no host launch cost between them) and rotate over enough
    copies of their buffers to cover 1 GiB, so no launch finds its inputs in
    the 256 MB last-level cache; the graph is replayed R times and the
    per-launch time is reported as median, p10 and p90 over the replays.
    Returns a list of records."""
    import torch

    import norm_rope_swiglu_amd as nrs
    import workloads as W

    cases = [("prefill_bf16", lambda: W.prefill(device=dev)),
             ("ragged_bf16", lambda: W.ragged(device=dev))]
    for dt in ("bf16", "f32"):
        for H in (512, 1024, 1536, 2048, 4096):
            cases.append((f"sweep_{dt}_h{H}", lambda dt=dt, H=H: W.sweep(device=dev, dtype=dt, hidden=H,
                                                                          head_dim=128, tokens=32768)))

    def time_op(op, w):
        L = w.layer
        s = 4 if w.dtype == "f32" else 2
        T, I = w.tokens, w.inter
        byts = algorithmic_bytes(op, T, w.hidden, I, w.n_q, w.n_kv, w.head_dim, s)
        nb = max(1, -(-(1 << 30) // byts))
        empty = lambda t: torch.empty_like(t)
        if op == "rmsnorm":
            sets = [(L.residual.clone(), empty(L.x)) for _ in range(nb)]
            fn = lambda b: nrs.rmsnorm(b[0], L.gamma, w.eps, out=b[1])
        elif op == "add_rmsnorm":
            sets = [(L.x.clone(), L.residual.clone(), empty(L.x), empty(L.x)) for _ in range(nb)]
            fn = lambda b: nrs.add_rmsnorm(b[0], b[1], L.gamma, w.eps, out=b[2], residual_out=b[3])
        elif op == "mrope":
            sets = [(L.q.clone(), L.k.clone()) for _ in range(nb)]
            fn = lambda b: nrs.mrope(b[0], b[1], w.pos, w.sections, w.theta)
        else:
            sets = [(L.gate_up.clone(), torch.empty(T, I, dtype=L.x.dtype, device=dev))
                    for _ in range(nb)]
            fn = lambda b: nrs.swiglu(b[0], out=b[1])
        for b in sets[:2]:
            fn(b)
        torch.cuda.synchronize()
        graph, gs = torch.cuda.CUDAGraph(), torch.cuda.Stream(dev)
        with torch.cuda.graph(graph, stream=gs):
            for i in range(K):
                fn(sets[i % nb])
        graph.replay()
        torch.cuda.synchronize()
        per, cur = [], torch.cuda.current_stream(dev)    # replays run on the current stream
        for _ in range(R):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(cur)
            graph.replay()
            b.record(cur)
            torch.cuda.synchronize()
            per.append(1e3 * a.elapsed_time(b) / K)
        per.sort()
        us = per[R // 2]
        del graph, sets
        torch.cuda.empty_cache()
        return {"us": round(us, 2), "p10_us": round(per[R // 10], 2),
                "p90_us": round(per[R - 1 - R // 10], 2), "buffer_sets": nb,
                "GB_s": round(byts / (us * 1e-6) / 1e9, 1),
                "frac_of_peak": round(byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}

    out = []
    for name, make in cases:
        if only and name not in only:
            continue
        w = make()
        rec = {"workload": name, "tokens": w.tokens, "hidden": w.hidden, "dtype": w.dtype,
               "head_dim": w.head_dim,
               "timing": f"graph of {K} launches over buffer copies covering 1 GiB, "
                         f"median/p10/p90 of {R} replays"}
        for op in ("rmsnorm", "add_rmsnorm", "mrope", "swiglu"):
            rec[op] = time_op(op, w)
        del w
        if name.startswith("sweep_"):
            # M-RoPE again at head_dim 64 (sections 8/12/12), the sweep's other head size
            w = W.sweep(device=dev, dtype=rec["dtype"], hidden=rec["hidden"], head_dim=64,
                        tokens=rec["tokens"])
            rec["mrope_head_dim64"] = time_op("mrope", w)
            del w
        out.append(rec)
        print("bench sweep: " + json.dumps(rec), file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-replays", type=int, default=500)
    ap.add_argument("--cpu-tokens", type=int, default=32768)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--sweep", metavar="FILE",
                    help="also time every op on every bandwidth-bound recipe, written to FILE as JSON")
    ap.add_argument("--sweep-only", metavar="NAME", action="append",
                    help="restrict --sweep to the named recipes (e.g. sweep_bf16_h2048); repeatable")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the ops are independent per token; see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import norm_rope_swiglu_amd as nrs
    import workloads as W

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    nrs.lib()

    # --- the step's batch, generated on the device.  rmsnorm gets its own
    # input rows so no op reads what the op before it just read.
    T, H, D = 32768, 2048, 128
    w = W.sweep(seed=0, device=dev, dtype="bf16", hidden=H, head_dim=D, tokens=T)
    L = w.layer
    xn = W.sweep(seed=1, device=dev, dtype="bf16", hidden=H, head_dim=D, tokens=T).layer.x
    I, nq, nkv = w.inter, w.n_q, w.n_kv
    s = 2
    y = torch.empty_like(L.x)
    y2 = torch.empty_like(L.x)
    ro = torch.empty_like(L.x)
    act = torch.empty(T, I, dtype=L.x.dtype, device=dev)
    q, k = L.q.clone(), L.k.clone()
    ops = ["rmsnorm", "add_rmsnorm", "mrope", "swiglu"]
    op_bytes = {op: algorithmic_bytes(op, T, H, I, nq, nkv, D, s) for op in ops}
    step_bytes = sum(op_bytes.values())

    def run(op):
        if op == "rmsnorm":
            nrs.rmsnorm(xn, L.gamma, w.eps, out=y)
        elif op == "add_rmsnorm":
            nrs.add_rmsnorm(L.x, L.residual, L.gamma, w.eps, out=y2, residual_out=ro)
        elif op == "mrope":
            nrs.mrope(q, k, w.pos, w.sections, w.theta)
        else:
            nrs.swiglu(L.gate_up, out=act)

    # calibration copy of known size (1 GiB), for the counter runs' scale factor
    src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    print(f"bench: warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for op in ops:
            run(op)
    torch.cuda.synchronize()

    # the timed steps: K passes of the four ops, back to back, one event pair
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(K):
        for op in ops:
            run(op)
    end.record(stream)
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / K

    # per-op launch duration: K launches of one op back to back between two
    # events (launch latency overlaps the previous launch, as in the step),
    # repeated NREP times; mean, median, p10 / p90 and extremes over the repeats
    per_op = {}
    NREP = 11
    for op in ops:
        reps = []
        for _ in range(NREP):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(K):
                run(op)
            b.record(stream)
            torch.cuda.synchronize()
            reps.append(1e3 * a.elapsed_time(b) / K)
        reps.sort()
        mean_us = sum(reps) / NREP
        gbs = op_bytes[op] / (mean_us * 1e-6) / 1e9
        per_op[op] = {"mean_us": round(mean_us, 2), "median_us": round(reps[NREP // 2], 2),
                      "p10_us": round(reps[NREP // 10], 2), "p90_us": round(reps[NREP - 1 - NREP // 10], 2),
                      "min_us": round(reps[0], 2), "max_us": round(reps[-1], 2), "bytes": op_bytes[op],
                      "GB_s": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
    print(f"bench: step {step_ms:.3f} ms; " + ", ".join(f"{o} {per_op[o]['mean_us']} us"
          for o in ops), file=sys.stderr, flush=True)

    # --- decode-step op set, hipGraph replay
    decode = None
    if not args.no_decode:
        dw = W.decode(seed=0, n_layers=28, second_norm=True)
        pos_d = dw.pos.to(dev)
        decode = {"workload": "5 sequences x 1 token, hidden 2048, q16/kv8 x 128, intermediate 6144, "
                              "28 layers, bf16"}
        for four_op in (False, True):
            bufs, R = [], dw.layers[0].residual.to(dev)
            for Ld in dw.layers:
                d = {"in_x": Ld.x.to(dev), "in_residual": R, "in_gamma": Ld.gamma.to(dev),
                     "in_y": torch.empty(5, 2048, dtype=torch.bfloat16, device=dev),
                     "in_residual_out": torch.empty(5, 2048, dtype=torch.bfloat16, device=dev),
                     "q": Ld.q.to(dev), "k": Ld.k.to(dev), "gate_up": Ld.gate_up.to(dev),
                     "act_out": torch.empty(5, 6144, dtype=torch.bfloat16, device=dev)}
                R = d["in_residual_out"]
                if four_op:
                    d.update(post_x=Ld.x2.to(dev), post_residual=R, post_gamma=Ld.gamma2.to(dev),
                             post_y=torch.empty_like(R), post_residual_out=torch.empty_like(R))
                    R = d["post_residual_out"]
                bufs.append(d)
            g = nrs.decode_graph(bufs, pos_d, dw.sections, dw.theta, dw.eps)
            floor = nrs.null_graph(g.nodes)
            res = {}
            for name, gr in (("op_set", g), ("empty_graph_same_nodes", floor)):
                for _ in range(20):
                    gr.launch(stream)
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(args.decode_replays):
                    gr.launch(stream)
                b.record(stream)
                torch.cuda.synchronize()
                res[name + "_us_per_step"] = round(1e3 * a.elapsed_time(b) / args.decode_replays, 2)
            per_layer = (algorithmic_bytes("add_rmsnorm", 5, 2048, 6144, 16, 8, 128, 2) * (2 if four_op else 1)
                         + algorithmic_bytes("mrope", 5, 2048, 6144, 16, 8, 128, 2)
                         + algorithmic_bytes("swiglu", 5, 2048, 6144, 16, 8, 128, 2))
            res.update(nodes=g.nodes, bytes_per_step=28 * per_layer)
            decode["four_op_layer" if four_op else "three_op_layer"] = res
            g.close()
            floor.close()
        print(f"bench: decode {json.dumps(decode)}", file=sys.stderr, flush=True)

    # --- ops beyond the four-op step, on the same batch
    next_ops = {}
    v = torch.empty_like(L.k).normal_()
    kc = torch.empty(1, nkv, T, D, dtype=L.k.dtype, device=dev)
    vc = torch.empty_like(kc)
    seq0 = torch.zeros(T, dtype=torch.int32, device=dev)
    slots = torch.arange(T, dtype=torch.int32, device=dev)
    # sampling: the decode step's 5 candidates over a 3072-entry codec vocabulary, and a
    # text-sized vocabulary at 256 rows (algorithmic bytes: logits read once, u, token)
    lg_dec = torch.randn(5, 3072, device=dev).mul_(4.0).to(torch.bfloat16)
    lg_big = torch.randn(256, 151936, device=dev).mul_(3.0).to(torch.bfloat16)
    u5, u256 = torch.rand(5, device=dev), torch.rand(256, device=dev)
    tok5 = torch.empty(5, dtype=torch.int32, device=dev)
    tok256 = torch.empty(256, dtype=torch.int32, device=dev)
    beta = torch.empty_like(L.gamma).normal_().mul_(0.1)
    nxt = {"layernorm": (lambda: nrs.layernorm(xn, L.gamma, beta, 1e-5, out=y),
                         algorithmic_bytes("layernorm", T, H, I, nq, nkv, D, s)),
           "add_layernorm": (lambda: nrs.add_layernorm(L.x, L.residual, L.gamma, beta, 1e-5, out=y2,
                                                       residual_out=ro),
                             algorithmic_bytes("add_layernorm", T, H, I, nq, nkv, D, s)),
           "mrope_kv_append": (lambda: nrs.mrope_kv_append(q, L.k, v, w.pos, w.sections, w.theta,
                                                           kc, vc, seq0, slots),
                               algorithmic_bytes("mrope_kv_append", T, H, I, nq, nkv, D, s)),
           "softmax_topk_sample_5x3072_k50": (
               lambda: nrs.softmax_topk_sample(lg_dec, 0.9, 50, u5, token=tok5), 5 * 3072 * 2 + 5 * 8),
           "softmax_topk_sample_256x151936_k50": (
               lambda: nrs.softmax_topk_sample(lg_big, 1.0, 50, u256, token=tok256),
               256 * 151936 * 2 + 256 * 8)}
    # fused RMSNorm + Linear at the decode step's projection shapes: 5 rows of 2048 into
    # qkv (4096) and gate_up (12288), one distinct weight per layer for 28 layers (so each
    # call streams its weight from HBM, 0.5-1.4 GB in all); recorded in a graph, so the
    # time per call has no host launch cost in it
    lin_x = torch.empty(5, H, device=dev).normal_().to(torch.bfloat16)
    lin = {}
    for n_out in (4096, 12288):
        ws = [torch.empty(n_out, H, device=dev).normal_().div_(45.0).to(torch.bfloat16)
              for _ in range(28)]
        yo = torch.empty(5, n_out, dtype=torch.bfloat16, device=dev)
        gs = torch.cuda.Stream(dev)
        with torch.cuda.stream(gs):
            for wt in ws:
                nrs.rmsnorm_linear(lin_x, wt, 1e-6, out=yo)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            for wt in ws:
                nrs.rmsnorm_linear(lin_x, wt, 1e-6, out=yo)
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(K):
            graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / (K * 28)
        byts = n_out * H * 2 + 5 * H * 2 + 5 * n_out * 2
        lin[f"rmsnorm_linear_5x2048x{n_out}_graph28"] = {
            "mean_us": round(us, 2), "bytes": byts, "GB_s": round(byts / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        del ws, graph
    # the decode-size sampler recorded in a graph (20 calls over distinct logits), so the time
    # per call has no host launch cost in it
    lgs = [torch.randn(5, 3072, device=dev).mul_(4.0).to(torch.bfloat16) for _ in range(20)]
    gs = torch.cuda.Stream(dev)
    with torch.cuda.stream(gs):
        for lg in lgs:
            nrs.softmax_topk_sample(lg, 0.9, 50, u5, token=tok5)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gs):
        for lg in lgs:
            nrs.softmax_topk_sample(lg, 0.9, 50, u5, token=tok5)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(K):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * a.elapsed_time(b) / (K * len(lgs))
    byts = 5 * 3072 * 2 + 5 * 8
    lin["softmax_topk_sample_5x3072_k50_graph20"] = {
        "mean_us": round(us, 2), "bytes": byts, "GB_s": round(byts / (us * 1e-6) / 1e9, 1),
        "frac_of_peak": round(byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    del lgs, graph
    # the prefill shape: 2048 tokens x 2048 -> 4096 (qkv), bound by the matrix cores
    lin_xp = torch.empty(2048, H, device=dev).normal_().to(torch.bfloat16)
    lin_wp = torch.empty(4096, H, device=dev).normal_().div_(45.0).to(torch.bfloat16)
    lin_yp = torch.empty(2048, 4096, dtype=torch.bfloat16, device=dev)
    nxt["rmsnorm_linear_2048x2048x4096"] = (
        lambda: nrs.rmsnorm_linear(lin_xp, lin_wp, 1e-6, out=lin_yp),
        2048 * H * 2 + 4096 * H * 2 + 2048 * 4096 * 2)
    for op, (fn, byts) in nxt.items():
        for _ in range(3):
            fn()
        reps = []
        for _ in range(NREP):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(K):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            reps.append(1e3 * a.elapsed_time(b) / K)
        mean_us = sum(reps) / NREP
        next_ops[op] = {"mean_us": round(mean_us, 2), "bytes": byts,
                        "GB_s": round(byts / (mean_us * 1e-6) / 1e9, 1),
                        "frac_of_peak": round(byts / (mean_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        if op.startswith("rmsnorm_linear_2048"):   # a contraction: priced against the bf16 MFMA peak
            tf = 2 * 2048 * H * 4096 / (mean_us * 1e-6) / 1e12
            next_ops[op] = {"mean_us": round(mean_us, 2), "TFLOP_s": round(tf, 1),
                            "frac_of_peak": round(tf / PEAK_MFMA_BF16_TFLOPS, 4),
                            "peak": "bf16 dense MFMA 2500 TFLOP/s"}
    next_ops.update(lin)
    del v, kc, vc, lg_dec, lg_big, lin_xp, lin_wp, lin_yp
    print(f"bench: next {json.dumps(next_ops)}", file=sys.stderr, flush=True)

    sw = per_op["swiglu"]
    achieved = sw["GB_s"]  # algorithmic bytes per launch / mean launch duration
    traffic = traffic_from_counters(op_bytes["swiglu"])
    roofline = {"bound": "hbm", "kernel": "swiglu_kernel<bf16>", "achieved": achieved,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic, "algorithmic_bytes_per_launch": op_bytes["swiglu"],
                "mean_launch_us": sw["mean_us"]}

    cpu = None
    if not args.no_cpu_baseline:
        print(f"bench: cpu baseline on {args.cpu_tokens} tokens", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_tokens)

    if args.sweep:
        recs = op_sweep(dev, only=args.sweep_only)
        with open(args.sweep, "w") as f:
            json.dump(recs, f, indent=1)

    value = step_bytes / (step_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "config": {"workload": "decoder-layer op set rmsnorm+add_rmsnorm+mrope+swiglu over 32768 "
                               "tokens, hidden 2048, q16/kv8 x 128, intermediate 6144, bf16",
                   "tokens": T, "hidden": H, "n_q_heads": nq, "n_kv_heads": nkv, "head_dim": D,
                   "intermediate": I, "sections": list(w.sections), "theta": w.theta,
                   "bytes_per_step": step_bytes, "parallelism": "single GPU"},
        "per_op": per_op, "decode": decode, "next_ops": next_ops, "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
