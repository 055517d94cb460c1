#!/usr/bin/env python3
"""Benchmark of the fused decoder-layer ops on one MI355X.

A step is one pass of the four memory-bound ops over one synthetic batch of
32768 tokens (hidden 2048, 16 q / 8 kv heads of 128, intermediate 6144, bf16):
rmsnorm -> add_rmsnorm -> mrope (in place) -> swiglu, inputs resident in HBM.
`value` is the algorithmic bytes of a step over its time (GB/s).  Beside it
the same run times the decode-step op set (5 tokens x 28 layers of
add_rmsnorm -> mrope -> swiglu, and the 4-op layer with the post-attention
norm) replayed from one hipGraph, plus an empty-kernel graph with the same
node count as the launch floor.  `configs` times every op on every
bandwidth-bound workload (the 2048-token prefill, the packed ragged batch,
and the 32768-token sweep at hidden 512-4096 in bf16 and fp32, M-RoPE also at
head_dim 64), each launch graph-timed over buffer copies covering 1 GiB so no
launch finds its inputs in the 256 MB last-level cache, beside the library's
calibration kernel (nrs_stream_probe) moving the same bytes in the same
read/write mix: `frac_of_ceiling`.  `ceilings` gives that kernel's rates at 1
GiB per stream.  `next_ops` times the ops built beside the step (LayerNorm,
M-RoPE + KV-cache append, softmax + top-k sampling, and RMSNorm + Linear at
the decode step's projection shapes and two prefill shapes).

Every duration is taken with HIP events recorded on the stream the kernels
run on.  The oracle (the fp64 C reference) is timed on a bounded sample of the
same batch on the host for the CPU baseline.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                       [--configs NAME ...] [--no-decode] [--no-next]
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
ROTATE_BYTES = 1 << 30
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


# Read and write streams of an op, for the calibration kernel of the same mix:
# (number of read streams, number of write streams, bytes per stream).
def stream_mix(op, T, H, I, nq, nkv, D, s):
    if op in ("rmsnorm", "layernorm"):
        return 1, 1, T * H * s
    if op in ("add_rmsnorm", "add_layernorm"):
        return 2, 2, T * H * s
    if op == "mrope":
        return 1, 1, T * (nq + nkv) * D * s
    if op == "swiglu":
        return 2, 1, T * I * s
    if op == "mrope_kv_append":
        return 1, 1, T * (nq + 2 * nkv) * D * s
    raise ValueError(op)


def time_graph(dev, fn, sets, K=20, R=11):
    """Per-launch duration of fn over rotating buffer sets: K launches
    (launch i on set i mod len(sets)) captured in one graph, so no host
    launch cost sits between them; the graph is replayed R times between HIP
    events on the replay stream.  Returns median, mean, p10 and p90 in us."""
    import torch

    for b in sets[:2]:
        fn(b)
    torch.cuda.synchronize()
    graph, gs = torch.cuda.CUDAGraph(), torch.cuda.Stream(dev)
    with torch.cuda.graph(graph, stream=gs):
        for i in range(K):
            fn(sets[i % len(sets)])
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
    del graph
    per.sort()
    return {"us": round(per[R // 2], 2), "mean_us": round(sum(per) / R, 2),
            "p10_us": round(per[R // 10], 2), "p90_us": round(per[R - 1 - R // 10], 2)}


def rotation(nbytes):
    """Buffer copies an op rotates over so that K launches touch >= 1 GiB of
    distinct memory: no launch finds its inputs in the 256 MB last-level
    cache (MALL)."""
    return max(1, -(-ROTATE_BYTES // max(1, nbytes)))


def ceiling(dev, n_read, n_write, nbytes, cache, K=20, R=11, row_bytes=0):
    """The calibration kernel (nrs_stream_probe) at a given read/write mix and
    size, rotated and timed exactly like the ops, fastest of its four
    patterns (two for row-granular copies of row_bytes rows); memoised in
    `cache`."""
    import torch

    import norm_rope_swiglu_amd as nrs

    key = (n_read, n_write, nbytes, row_bytes)
    if key not in cache:
        nb = rotation(nbytes * (n_read + n_write))
        mk = lambda: torch.empty(nbytes, dtype=torch.uint8, device=dev)
        sets = []
        for _ in range(nb):
            src = [mk().fill_(0x11) for _ in range(n_read)]
            sets.append((src, [mk() for _ in range(n_write)]))
        best, per_variant = None, {}
        for v in range(2 if row_bytes else 4):
            t = time_graph(dev, lambda b, v=v: nrs.stream_probe(n_read, n_write, b[0], b[1], nbytes, v,
                                                                row_bytes=row_bytes),
                           sets, K, R)
            per_variant[v] = t["us"]
            if best is None or t["us"] < best["us"]:
                best = dict(t, variant=v)
        t = best
        moved = nbytes * (n_read + n_write)
        t.update(pattern=f"{n_read} read + {n_write} write streams of {nbytes} B"
                         + (f" in rows of {row_bytes} B" if row_bytes else ""),
                 GB_s=round(moved / (t["us"] * 1e-6) / 1e9, 1), buffer_sets=nb,
                 us_by_variant=per_variant)
        cache[key] = t
        del sets
        torch.cuda.empty_cache()
    return cache[key]


def op_runner(op, w, dev):
    """(launch function over one buffer set, buffer sets) for one op of a
    workload; the sets cover >= 1 GiB together (see rotation)."""
    import torch

    import norm_rope_swiglu_amd as nrs

    L = w.layer
    s = 4 if w.dtype == "f32" else 2
    byts = algorithmic_bytes(op, w.tokens, w.hidden, w.inter, w.n_q, w.n_kv, w.head_dim, s)
    nb = rotation(byts)
    empty = torch.empty_like
    if op == "rmsnorm":
        sets = [(L.residual.clone(), empty(L.x)) for _ in range(nb)]
        return (lambda b: nrs.rmsnorm(b[0], L.gamma, w.eps, out=b[1])), sets, byts
    if op == "add_rmsnorm":
        sets = [(L.x.clone(), L.residual.clone(), empty(L.x), empty(L.x)) for _ in range(nb)]
        return (lambda b: nrs.add_rmsnorm(b[0], b[1], L.gamma, w.eps, out=b[2], residual_out=b[3])), sets, byts
    if op == "mrope":
        sets = [(L.q.clone(), L.k.clone()) for _ in range(nb)]
        return (lambda b: nrs.mrope(b[0], b[1], w.pos, w.sections, w.theta)), sets, byts
    if op == "swiglu":
        sets = [(L.gate_up.clone(), torch.empty(w.tokens, w.inter, dtype=L.x.dtype, device=dev))
                for _ in range(nb)]
        return (lambda b: nrs.swiglu(b[0], out=b[1])), sets, byts
    raise ValueError(op)


def measure_op(dev, op, w, ceil_cache, K=20, R=11):
    """One op on one workload: graph-timed with rotation, beside the
    calibration kernel of the same read/write mix and size."""
    import torch

    fn, sets, byts = op_runner(op, w, dev)
    t = time_graph(dev, fn, sets, K, R)
    del sets
    torch.cuda.empty_cache()
    s = 4 if w.dtype == "f32" else 2
    nr, nw, nbytes = stream_mix(op, w.tokens, w.hidden, w.inter, w.n_q, w.n_kv, w.head_dim, s)
    c = ceiling(dev, nr, nw, nbytes, ceil_cache, K, R)
    gbs = byts / (t["us"] * 1e-6) / 1e9
    t.update(bytes=byts, GB_s=round(gbs, 1), frac_of_peak=round(gbs / PEAK_HBM_GBS, 4),
             ceiling_us=c["us"], ceiling_GB_s=c["GB_s"],
             frac_of_ceiling=round(c["us"] / t["us"], 4))
    rb = row_ceiling_bytes(op, w.hidden, s)
    if rb:
        # a single-pass norm holds a row per workgroup: the ceiling of that access
        # pattern is the row-granular copy of the same rows and mix
        rc = ceiling(dev, nr, nw, nbytes, ceil_cache, K, R, row_bytes=rb)
        t.update(row_ceiling_us=rc["us"], row_ceiling_GB_s=rc["GB_s"],
                 frac_of_row_ceiling=round(rc["us"] / t["us"], 4))
    return t


def row_ceiling_bytes(op, H, s):
    """Row size of the row-granular calibration copy that matches a norm op
    (0: none; the calibration kernel builds rows of 1-4, 6, 8, 12, 16 KiB)."""
    if op not in ("rmsnorm", "add_rmsnorm", "layernorm", "add_layernorm"):
        return 0
    rb = H * s
    return rb if rb % 1024 == 0 and (rb >> 10) in (1, 2, 3, 4, 6, 8, 12, 16) else 0


def config_cases(dev):
    """The bandwidth-bound workloads: the 2048-token prefill, the packed ragged
    batch, and the 32768-token sweep at every width and dtype (head_dim 128;
    M-RoPE again at head_dim 64)."""
    import workloads as W

    cases = [("prefill_bf16", lambda: W.prefill(device=dev)),
             ("ragged_bf16", lambda: W.ragged(device=dev))]
    for dt in ("bf16", "f32"):
        for H in (512, 1024, 1536, 2048, 4096):
            cases.append((f"sweep_{dt}_h{H}", lambda dt=dt, H=H: W.sweep(
                device=dev, dtype=dt, hidden=H, head_dim=128, tokens=32768)))
    return cases


def measure_configs(dev, ceil_cache, only=None, reuse=None, K=20, R=11):
    """Every op on every bandwidth-bound workload (config_cases).  `reuse`
    maps a case name to an already generated workload."""
    import torch

    import workloads as W

    out = []
    for name, make in config_cases(dev):
        if only and name not in only:
            continue
        w = (reuse or {}).get(name) or make()
        rec = {"workload": name, "tokens": w.tokens, "hidden": w.hidden, "inter": w.inter,
               "dtype": w.dtype, "head_dim": w.head_dim, "n_q": w.n_q, "n_kv": w.n_kv,
               "timing": f"graph of {K} launches over buffer copies covering >= 1 GiB, "
                         f"median/p10/p90 of {R} replays; ceiling: nrs_stream_probe at the "
                         "op's read/write mix and size, timed the same way"}
        for op in ("rmsnorm", "add_rmsnorm", "mrope", "swiglu"):
            rec[op] = measure_op(dev, op, w, ceil_cache, K, R)
        del w
        torch.cuda.empty_cache()
        if name.startswith("sweep_"):
            # M-RoPE again at head_dim 64 (sections 8/12/12), the sweep's other head size
            w = W.sweep(device=dev, dtype=rec["dtype"], hidden=rec["hidden"], head_dim=64,
                        tokens=rec["tokens"])
            rec["mrope_head_dim64"] = measure_op(dev, "mrope", w, ceil_cache, K, R)
            del w
            torch.cuda.empty_cache()
        out.append(rec)
        print("bench config: " + json.dumps(rec), file=sys.stderr, flush=True)
    return out


def bar_summary(configs, bar=0.8):
    """Which (workload, op) pairs sit below `bar` of the HBM peak, and the
    lowest fraction of the matched calibration kernel."""
    below, worst = [], None
    for rec in configs:
        for op in ("rmsnorm", "add_rmsnorm", "mrope", "swiglu", "mrope_head_dim64"):
            r = rec.get(op)
            if r is None:
                continue
            if r["frac_of_peak"] < bar:
                b = {"workload": rec["workload"], "op": op, "frac_of_peak": r["frac_of_peak"],
                     "frac_of_ceiling": r["frac_of_ceiling"],
                     "ceiling_frac_of_peak": round(r["ceiling_GB_s"] / PEAK_HBM_GBS, 4)}
                if "row_ceiling_GB_s" in r:
                    b.update(frac_of_row_ceiling=r["frac_of_row_ceiling"],
                             row_ceiling_frac_of_peak=round(r["row_ceiling_GB_s"] / PEAK_HBM_GBS, 4))
                below.append(b)
            if worst is None or r["frac_of_ceiling"] < worst["frac_of_ceiling"]:
                worst = {"workload": rec["workload"], "op": op, "frac_of_ceiling": r["frac_of_ceiling"]}
    n = sum(1 for rec in configs for op in ("rmsnorm", "add_rmsnorm", "mrope", "swiglu",
                                             "mrope_head_dim64") if op in rec)
    return {"bar": bar, "pairs": n, "pairs_below_bar": len(below), "below": below,
            "lowest_frac_of_ceiling": worst}


def eager_time(dev, fn, K):
    """Mean microseconds of fn over K launches queued back to back after three
    warm-up calls, bracketed by events on the current stream."""
    import torch

    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream(dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(cur)
    for _ in range(K):
        fn()
    b.record(cur)
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / K


def measure_next(dev, w, ceil_cache, K=20, R=11):
    """The ops built beside the four-op step, on the step's batch shapes:
    LayerNorm (plain and fused), M-RoPE + KV-cache append and the sampler over
    a text-sized vocabulary (graph-timed with rotation, beside the matched
    calibration kernel); the decode-size sampler and RMSNorm + Linear at the
    decode step's projection shapes (graphs of distinct inputs); the prefill
    RMSNorm + Linear, priced against the bf16 matrix-core peak."""
    import torch

    import norm_rope_swiglu_amd as nrs

    L = w.layer
    T, H, I, nq, nkv, D, s = w.tokens, w.hidden, w.inter, w.n_q, w.n_kv, w.head_dim, 2
    res = {}

    def rotated(name, fn, sets, byts, mix, row_bytes=0, row_pattern=None):
        t = time_graph(dev, fn, sets, K, R)
        gbs = byts / (t["us"] * 1e-6) / 1e9
        t.update(bytes=byts, GB_s=round(gbs, 1), frac_of_peak=round(gbs / PEAK_HBM_GBS, 4))
        if mix is not None:
            c = ceiling(dev, *mix, ceil_cache, K, R)
            t.update(ceiling_us=c["us"], ceiling_GB_s=c["GB_s"],
                     frac_of_ceiling=round(c["us"] / t["us"], 4))
        if row_bytes:
            rc = ceiling(dev, *mix, ceil_cache, K, R, row_bytes=row_bytes)
            t.update(row_ceiling_us=rc["us"], row_ceiling_GB_s=rc["GB_s"],
                     frac_of_row_ceiling=round(rc["us"] / t["us"], 4))
            if row_pattern:
                t.update(row_ceiling_pattern=row_pattern)
        res[name] = t
        torch.cuda.empty_cache()

    beta = torch.empty_like(L.gamma).normal_().mul_(0.1)
    byts = algorithmic_bytes("layernorm", T, H, I, nq, nkv, D, s)
    sets = [(L.residual.clone(), torch.empty_like(L.x)) for _ in range(rotation(byts))]
    rotated("layernorm", lambda b: nrs.layernorm(b[0], L.gamma, beta, 1e-5, out=b[1]), sets, byts,
            stream_mix("layernorm", T, H, I, nq, nkv, D, s), row_ceiling_bytes("layernorm", H, s))
    byts = algorithmic_bytes("add_layernorm", T, H, I, nq, nkv, D, s)
    sets = [(L.x.clone(), L.residual.clone(), torch.empty_like(L.x), torch.empty_like(L.x))
            for _ in range(rotation(byts))]
    rotated("add_layernorm", lambda b: nrs.add_layernorm(b[0], b[1], L.gamma, beta, 1e-5, out=b[2],
                                                         residual_out=b[3]),
            sets, byts, stream_mix("add_layernorm", T, H, I, nq, nkv, D, s),
            row_ceiling_bytes("add_layernorm", H, s))
    del sets
    # M-RoPE + KV-cache append: one 32768-slot sequence, slot = token index
    byts = algorithmic_bytes("mrope_kv_append", T, H, I, nq, nkv, D, s)
    seq0 = torch.zeros(T, dtype=torch.int32, device=dev)
    slots = torch.arange(T, dtype=torch.int32, device=dev)
    sets = []
    for _ in range(rotation(byts)):
        kc = torch.empty(1, nkv, T, D, dtype=L.k.dtype, device=dev)
        sets.append((L.q.clone(), L.k.clone(), torch.empty_like(L.k).normal_(), kc, torch.empty_like(kc)))
    rotated("mrope_kv_append", lambda b: nrs.mrope_kv_append(b[0], b[1], b[2], w.pos, w.sections,
                                                             w.theta, b[3], b[4], seq0, slots),
            sets, byts, stream_mix("mrope_kv_append", T, H, I, nq, nkv, D, s))
    del sets
    # the same append for a 2048-token prefill (the first 2048 tokens, a 2048-slot cache)
    Tp = 2048
    byts = algorithmic_bytes("mrope_kv_append", Tp, H, I, nq, nkv, D, s)
    sets = []
    for _ in range(rotation(byts)):
        kc = torch.empty(1, nkv, Tp, D, dtype=L.k.dtype, device=dev)
        sets.append((L.q[:Tp].clone(), L.k[:Tp].clone(), torch.empty_like(L.k[:Tp]).normal_(), kc,
                     torch.empty_like(kc)))
    rotated("mrope_kv_append_prefill2048",
            lambda b: nrs.mrope_kv_append(b[0], b[1], b[2], w.pos, w.sections, w.theta, b[3], b[4],
                                          seq0[:Tp], slots[:Tp]),
            sets, byts, stream_mix("mrope_kv_append", Tp, H, I, nq, nkv, D, s))
    del sets
    # sampling over a text-sized vocabulary: 256 rows x 151936 bf16 logits (algorithmic
    # bytes: the logits read once, u read and the token written); ceilings: the flat
    # read-only kernel over the logits, and the row-granular read of the sampler's own
    # shape (one 1024-thread workgroup per row, reading it and nothing else)
    byts = 256 * 151936 * 2 + 256 * 8
    sets = [(torch.randn(256, 151936, device=dev).mul_(3.0).to(torch.bfloat16),
             torch.rand(256, device=dev), torch.empty(256, dtype=torch.int32, device=dev))
            for _ in range(rotation(byts))]
    rotated("softmax_topk_sample_256x151936_k50",
            lambda b: nrs.softmax_topk_sample(b[0], 1.0, 50, b[1], token=b[2]), sets, byts,
            (1, 0, 256 * 151936 * 2), row_bytes=151936 * 2,
            row_pattern="read only: one 1024-thread workgroup per 303872-byte row")
    del sets

    # decode-size calls recorded in graphs over distinct inputs (so no host launch cost and
    # every call streams its own weights / logits)
    def graph_calls(name, calls, byts, n):
        gs = torch.cuda.Stream(dev)
        with torch.cuda.stream(gs):
            for c in calls:
                c()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            for c in calls:
                c()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream(dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(cur)
        for _ in range(K):
            graph.replay()
        b.record(cur)
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / (K * n)
        res[name] = {"mean_us": round(us, 2), "bytes": byts, "GB_s": round(byts / (us * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        del graph

    lin_x = torch.empty(5, H, device=dev).normal_().to(torch.bfloat16)
    for n_out in (4096, 12288):
        ws = [torch.empty(n_out, H, device=dev).normal_().div_(45.0).to(torch.bfloat16)
              for _ in range(28)]
        yo = torch.empty(5, n_out, dtype=torch.bfloat16, device=dev)
        name = f"rmsnorm_linear_5x2048x{n_out}_graph28"
        graph_calls(name, [lambda wt=wt: nrs.rmsnorm_linear(lin_x, wt, 1e-6, out=yo) for wt in ws],
                    n_out * H * 2 + 5 * H * 2 + 5 * n_out * 2, 28)
        # the read-only calibration kernel over the same 28 weights, recorded the same way:
        # the fastest a kernel that only reads each weight once can go at this size
        best = None
        for v in range(4):
            graph_calls("_ceiling", [lambda wt=wt, v=v: nrs.stream_probe(1, 0, [wt], [], None, v)
                                     for wt in ws], n_out * H * 2, 28)
            c = res.pop("_ceiling")
            best = c if best is None or c["mean_us"] < best["mean_us"] else best
        res[name].update(ceiling_us=best["mean_us"], ceiling_GB_s=best["GB_s"],
                         frac_of_ceiling=round(best["mean_us"] / res[name]["mean_us"], 4))
        del ws
    u5 = torch.rand(5, device=dev)
    tok5 = torch.empty(5, dtype=torch.int32, device=dev)
    lgs = [torch.randn(5, 3072, device=dev).mul_(4.0).to(torch.bfloat16) for _ in range(20)]
    graph_calls("softmax_topk_sample_5x3072_k50_graph20",
                [lambda lg=lg: nrs.softmax_topk_sample(lg, 0.9, 50, u5, token=tok5) for lg in lgs],
                5 * 3072 * 2 + 5 * 8, 20)
    del lgs

    # the prefill projections, bound by the matrix cores
    for M, N in ((2048, 4096), (32768, 4096)):
        xp = torch.empty(M, H, device=dev).normal_().to(torch.bfloat16)
        wp = torch.empty(N, H, device=dev).normal_().div_(45.0).to(torch.bfloat16)
        yp = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        t = time_graph(dev, lambda b: nrs.rmsnorm_linear(b[0], b[1], 1e-6, out=b[2]), [(xp, wp, yp)],
                       K, R)
        tf = 2 * M * H * N / (t["mean_us"] * 1e-6) / 1e12
        t.update(TFLOP_s=round(tf, 1), frac_of_peak=round(tf / PEAK_MFMA_BF16_TFLOPS, 4),
                 peak="bf16 dense MFMA 2500 TFLOP/s")
        # the vendor library's plain product of the same operands (no norm), for a
        # practical ceiling: torch.mm on a contiguous W^T, launched eagerly (a library
        # call may record memsets, which stay out of graphs)
        wt = wp.t().contiguous()
        lib_us = eager_time(dev, lambda: torch.mm(xp, wt, out=yp), K)
        ltf = 2 * M * H * N / (lib_us * 1e-6) / 1e12
        t.update(library_us=round(lib_us, 2), library_TFLOP_s=round(ltf, 1),
                 frac_of_library=round(lib_us / t["mean_us"], 4), library="torch.mm (hipBLASLt)")
        res[f"rmsnorm_linear_{M}x{H}x{N}"] = t
        del xp, wp, yp, wt
    torch.cuda.empty_cache()
    print(f"bench: next {json.dumps(res)}", file=sys.stderr, flush=True)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-replays", type=int, default=500)
    ap.add_argument("--cpu-tokens", type=int, default=32768)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the ops beyond the four-op step")
    ap.add_argument("--configs", metavar="NAME", action="append",
                    help="time only the named bandwidth-bound workloads (e.g. sweep_bf16_h2048, "
                         "prefill_bf16); repeatable; 'none' skips them")
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
    print(f"bench: step {step_ms:.3f} ms", file=sys.stderr, flush=True)
    del y, y2, ro, act, q, k, xn
    torch.cuda.empty_cache()

    # --- calibration: the streaming kernel at 1 GiB per stream, each mix
    ceil_cache = {}
    ceilings = {}
    for name, (nr, nw) in (("read", (1, 0)), ("write", (0, 1)), ("copy", (1, 1)),
                           ("read2_write1", (2, 1)), ("read2_write2", (2, 2))):
        c = ceiling(dev, nr, nw, 1 << 30, ceil_cache)
        ceilings[name] = {"GB_s": c["GB_s"], "frac_of_peak": round(c["GB_s"] / PEAK_HBM_GBS, 4),
                          "us": c["us"], "bytes_per_stream": 1 << 30}
    print(f"bench: ceilings {json.dumps(ceilings)}", file=sys.stderr, flush=True)

    # --- every op on every bandwidth-bound workload (the headline shape is
    # sweep_bf16_h2048, whose per-op figures are the per_op block)
    only = args.configs
    if only is None or only != ["none"]:
        configs = measure_configs(dev, ceil_cache, only=only, reuse={"sweep_bf16_h2048": w})
    else:
        configs = []
    head = next((r for r in configs if r["workload"] == "sweep_bf16_h2048"), None)
    if head is None:     # not among the selected workloads: time the headline ops alone
        head = {op: measure_op(dev, op, w, ceil_cache) for op in ops}
    per_op = {op: head[op] for op in ops}
    print("bench: per-op " + ", ".join(f"{o} {per_op[o]['us']} us" for o in ops),
          file=sys.stderr, flush=True)

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

    next_ops = None if args.no_next else measure_next(dev, w, ceil_cache, K)

    sw = per_op["swiglu"]
    achieved = op_bytes["swiglu"] / (sw["mean_us"] * 1e-6) / 1e9  # algorithmic bytes / mean launch
    traffic = traffic_from_counters(op_bytes["swiglu"])
    roofline = {"bound": "hbm", "kernel": "swiglu_kernel<bf16>", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic, "algorithmic_bytes_per_launch": op_bytes["swiglu"],
                "mean_launch_us": sw["mean_us"],
                "launch_timing": "graph of 20 launches over buffer copies covering >= 1 GiB, "
                                 "mean of 11 replays, HIP events on the replay stream",
                "ceiling_GB_s": sw["ceiling_GB_s"], "frac_of_ceiling": sw["frac_of_ceiling"]}

    cpu = None
    if not args.no_cpu_baseline:
        print(f"bench: cpu baseline on {args.cpu_tokens} tokens", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_tokens)

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
        "per_op": per_op, "ceilings": ceilings, "configs": configs,
        "bar_80": bar_summary(configs) if configs else None,
        "decode": decode, "next_ops": next_ops, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
