"""Full-size parity: every row of the benchmark's 32768-token launches.

The four ops run once over the whole batch on the GPU, in the launch
configuration bench.py times; every row of every output is then compared with
the oracle, which runs over row chunks on host threads (its C functions keep
no state and ctypes releases the GIL around them).  Workloads: the benchmark
step's batch (hidden 2048, 16 q / 8 kv heads of 128, bf16), the largest
sweep point (hidden 4096 fp32: 4.8 GB of SwiGLU input), the scaled-row sweep
at hidden 2048 with eps 1e-5, and M-RoPE at head_dim 64 on the sweep's
32 q / 16 kv heads (the 32768-token shape of the head_dim-64 kernel path).
Beside them, two ops beyond the four at the same batch: LayerNorm (plain and
with the residual add) and M-RoPE with the KV-cache append, every row.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import norm_rope_swiglu_amd as nrs
import oracle
import workloads as W
from numerics import ln_scale
from parity import check, check_exact

pytestmark = pytest.mark.gpu

CHUNK = 2048
THREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    nrs.lib()


def _f32(v):
    return float(np.float32(v))


def _over_chunks(T, job):
    spans = [(a, min(a + CHUNK, T)) for a in range(0, T, CHUNK)]
    with ThreadPoolExecutor(THREADS) as ex:
        for _ in ex.map(lambda ab: job(*ab), spans):
            pass
    return len(spans)


def full_layer_parity(w: W.Workload, tag: str, ops=("rmsnorm", "add_rmsnorm", "mrope", "swiglu")):
    L = w.layer
    T = w.tokens
    eps = _f32(w.eps)
    out = {}
    if "rmsnorm" in ops:
        out["rmsnorm"] = nrs.rmsnorm(L.x, L.gamma, w.eps)
    if "add_rmsnorm" in ops:
        out["add_y"], out["add_ro"] = nrs.add_rmsnorm(L.x, L.residual, L.gamma, w.eps)
    if "mrope" in ops:
        q, k = L.q.clone(), L.k.clone()
        nrs.mrope(q, k, w.pos, w.sections, w.theta)
        out["q"], out["k"] = q, k
    if "swiglu" in ops:
        out["swiglu"] = nrs.swiglu(L.gate_up)
    torch.cuda.synchronize()
    host = {n: t.cpu() for n, t in out.items()}
    del out
    x, res, gamma = L.x.cpu(), L.residual.cpu(), L.gamma.cpu()
    q0, k0, pos = (L.q.cpu(), L.k.cpu(), w.pos.cpu()) if "mrope" in ops else (None, None, None)
    gu = L.gate_up.cpu() if "swiglu" in ops else None

    def job(a, b):
        sl = slice(a, b)
        where = f"[{a}:{b}]"
        if "rmsnorm" in ops:
            check(f"{tag}/rmsnorm{where}", host["rmsnorm"][sl], oracle.rmsnorm(x[sl], gamma, eps))
        if "add_rmsnorm" in ops:
            ry, rro = oracle.add_rmsnorm(x[sl], res[sl], gamma, eps)
            check_exact(f"{tag}/add_rmsnorm.residual_out{where}", host["add_ro"][sl], rro)
            check(f"{tag}/add_rmsnorm.y{where}", host["add_y"][sl], ry)
        if "mrope" in ops:
            rq, rk = oracle.mrope(q0[sl], k0[sl], pos[:, sl].contiguous(), w.sections, w.theta)
            check(f"{tag}/mrope.q{where}", host["q"][sl], rq, pairs=True)
            check(f"{tag}/mrope.k{where}", host["k"][sl], rk, pairs=True)
        if "swiglu" in ops:
            check(f"{tag}/swiglu{where}", host["swiglu"][sl], oracle.swiglu(gu[sl]))

    n = _over_chunks(T, job)
    assert n * CHUNK >= T


def test_benchmark_batch_every_row():
    # the benchmark step's batch: 32768 tokens, hidden 2048, 16 q / 8 kv x 128, bf16
    w = W.sweep(seed=0, device="cuda", dtype="bf16", hidden=2048, head_dim=128, tokens=32768)
    full_layer_parity(w, "full/bf16/h2048")


def test_largest_sweep_point_every_row():
    # hidden 4096 fp32, intermediate 12288: the largest single-GPU sweep configuration
    w = W.sweep(device="cuda", dtype="f32", hidden=4096, head_dim=128, tokens=32768)
    full_layer_parity(w, "full/f32/h4096")


def test_scaled_rows_every_row():
    w = W.sweep(device="cuda", dtype="bf16", hidden=2048, head_dim=128, tokens=32768, scaled=True,
                eps=1e-5)
    full_layer_parity(w, "full_scaled/bf16/h2048")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mrope_head_dim64_sweep_shape_every_row(dtype):
    # 32 q / 16 kv heads of 64 (hidden 2048), sections 8/12/12, positions 0..32767
    w = W.sweep(device="cuda", dtype=dtype, hidden=2048, head_dim=64, tokens=32768)
    full_layer_parity(w, f"full_d64/{dtype}/h2048", ops=("mrope",))


def test_layernorm_every_row():
    # LayerNorm and the residual add + LayerNorm on the benchmark batch, with a beta
    w = W.sweep(seed=0, device="cuda", dtype="bf16", hidden=2048, head_dim=128, tokens=32768)
    L = w.layer
    beta = W.store(0.1 * W.normal(W.stream_key(0, "fullsize/ln/beta"), w.hidden), "bf16").cuda()
    eps = 1e-5
    y = nrs.layernorm(L.x, L.gamma, beta, eps)
    y2, ro = nrs.add_layernorm(L.x, L.residual, L.gamma, beta, eps)
    torch.cuda.synchronize()
    y, y2, ro = y.cpu(), y2.cpu(), ro.cpu()
    x, res, gamma, b = L.x.cpu(), L.residual.cpu(), L.gamma.cpu(), beta.cpu()
    gw, bw = oracle.widen(gamma), oracle.widen(b)
    e32 = _f32(eps)

    def job(a, c):
        sl = slice(a, c)
        where = f"[{a}:{c}]"
        xs = x[sl].contiguous()
        sc = ln_scale(oracle.widen(xs).reshape(xs.shape), gw, bw, e32)
        check(f"full/ln/y{where}", y[sl], oracle.layernorm(xs, gamma, b, e32), scale=sc)
        ry, h = oracle.add_layernorm(xs, res[sl].contiguous(), gamma, b, e32)
        check_exact(f"full/add_ln/residual_out{where}", ro[sl], h)
        sc = ln_scale(oracle.widen(h).reshape(h.shape), gw, bw, e32)
        check(f"full/add_ln/y{where}", y2[sl], ry, scale=sc)

    assert _over_chunks(w.tokens, job) * CHUNK >= w.tokens


def test_kv_append_every_token():
    # M-RoPE + KV-cache append on the benchmark batch's q and k (v drawn here), one
    # 32768-slot sequence with slots in reverse order: q, every k-cache and v-cache row
    w = W.sweep(seed=0, device="cuda", dtype="bf16", hidden=2048, head_dim=128, tokens=32768)
    L = w.layer
    T, nkv, D = L.k.shape
    g = torch.Generator().manual_seed(21)
    v = torch.randn(L.k.shape, generator=g, dtype=torch.float64).to(torch.float32).to(L.k.dtype).cuda()
    q = L.q.clone()
    kc = torch.full((1, nkv, T, D), -7.0, dtype=L.k.dtype, device="cuda")
    vc = torch.full_like(kc, -7.0)
    slot = torch.arange(T - 1, -1, -1, dtype=torch.int32, device="cuda")
    nrs.mrope_kv_append(q, L.k, v, w.pos, w.sections, w.theta, kc, vc,
                        torch.zeros(T, dtype=torch.int32, device="cuda"), slot)
    torch.cuda.synchronize()
    qh, kch, vch = q.cpu(), kc[0].cpu(), vc[0].cpu()
    q0, k0, v0, pos = L.q.cpu(), L.k.cpu(), v.cpu(), w.pos.cpu()

    def job(a, c):
        sl = slice(a, c)
        n = c - a
        where = f"[{a}:{c}]"
        rq, rkc, rvc = oracle.mrope_kv_append(
            q0[sl], k0[sl], v0[sl], pos[:, sl].contiguous(), w.sections, w.theta,
            torch.arange(n, dtype=torch.int32), torch.zeros(n, dtype=torch.int32),
            np.zeros((n, nkv, 1, D)), torch.zeros(n, nkv, 1, D, dtype=L.k.dtype))
        s = torch.arange(T - 1 - a, T - 1 - c, -1)               # slots of tokens a..c-1
        check(f"full/kv/q{where}", qh[sl], rq, pairs=True)
        check(f"full/kv/k_cache{where}", kch[:, s, :].permute(1, 0, 2), rkc[:, :, 0, :], pairs=True)
        check_exact(f"full/kv/v_cache{where}", vch[:, s, :].permute(1, 0, 2).contiguous(),
                    rvc[:, :, 0, :])

    assert _over_chunks(T, job) * CHUNK >= T
