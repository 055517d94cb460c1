"""The seeded input generators (CPU only): published SplitMix64 values,
Box-Muller structure, determinism, and the workload recipes."""
from __future__ import annotations

import math

import numpy as np
import torch

import workloads as W
from workloads import gen


def test_splitmix64_published_sequence():
    # Reference splitmix64.c seeded with 0 (Steele, Lea and Flood, OOPSLA 2014;
    # the C reference by S. Vigna) starts with these three outputs.
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert gen.splitmix64_int(0, 3) == want
    got = [v & (2**64 - 1) for v in gen.raw64(0, 0, 3, "cpu").tolist()]
    assert got == want


def test_counter_based_ranges_agree():
    key = gen.stream_key(7, "x")
    full = gen.normal(key, 1001)
    assert torch.equal(full[333:777], gen.normal(key, 444, start=333))
    assert torch.equal(gen.uniform(key, 50)[10:20], gen.uniform(key, 10, start=10))


def test_box_muller_pair():
    key = gen.stream_key(0, "bm")
    r = [v & (2**64 - 1) for v in gen.raw64(key, 0, 2, "cpu").tolist()]
    u1 = 1.0 - (r[0] >> 11) * 2.0**-53
    u2 = (r[1] >> 11) * 2.0**-53
    rad = math.sqrt(-2 * math.log(u1))
    n = gen.normal(key, 2)
    assert n[0].item() == rad * math.cos(2 * math.pi * u2)
    assert n[1].item() == rad * math.sin(2 * math.pi * u2)


def test_normal_moments():
    n = gen.normal(gen.stream_key(1, "m"), 400000).numpy()
    assert abs(n.mean()) < 5 / math.sqrt(4e5)
    assert abs(n.var() - 1) < 5 * math.sqrt(2 / 4e5)
    assert abs(np.mean(np.abs(n) > 1.96) - 0.05) < 0.002


def test_tiny_recipe():
    w = W.tiny()
    L = w.layer
    assert w.dtype == "f32" and L.x.dtype == torch.float32
    assert L.q.shape == (8, 4, 64) and L.k.shape == (8, 2, 64) and L.gate_up.shape == (8, 1536)
    assert w.pos.tolist() == [list(range(8))] * 3
    assert w.sections == (8, 12, 12) and sum(w.sections) == 32
    assert abs(L.gamma.mean().item() - 1) < 0.03


def test_decode_recipe_deterministic():
    a, b = W.decode(n_layers=2), W.decode(n_layers=2)
    assert torch.equal(a.layers[1].x, b.layers[1].x)
    assert not torch.equal(a.layers[0].gamma, a.layers[1].gamma)   # distinct gamma per layer
    p = a.pos
    assert torch.equal(p[0], p[1]) and torch.equal(p[0], p[2])
    assert p.min() >= 100 and p.max() <= 1500 and a.tokens == 5
    assert a.layer.x.dtype == torch.bfloat16 and a.sections == (16, 24, 24)


def test_prefill_positions_rule():
    p = W.prefill_positions(2048)
    assert p[:, :512].tolist() == [list(range(512))] * 3
    n = torch.arange(512, 2048)
    assert torch.equal(p[0, 512:], (512 + (n - 512) // 64).to(torch.int32))
    assert torch.equal(p[1, 512:], ((n - 512) % 64).to(torch.int32))
    assert torch.equal(p[1], p[2])


def test_ragged_recipe():
    lens = W.ragged_lengths(0)
    assert len(lens) == 64 and min(lens) >= 32 and max(lens) <= 1024
    w = W.ragged(n_seqs=6, hidden=256, head_dim=64)
    assert w.tokens == sum(w.seq_lens) and w.pos.shape == (3, w.tokens)
    start = 0
    for L in w.seq_lens:   # positions run consecutively within each sequence
        seg = w.pos[0, start:start + L]
        assert torch.equal(seg - seg[0], torch.arange(L, dtype=torch.int32))
        assert 0 <= seg[0] <= 1500
        start += L


def test_sweep_recipe_and_scales():
    w = W.sweep(dtype="f32", hidden=512, head_dim=64, tokens=64, scaled=True)
    assert (w.n_q, w.n_kv, w.inter, w.sections) == (8, 4, 1536, (8, 12, 12))
    rms = w.layer.x.double().pow(2).mean(1).sqrt()
    assert rms.min() < 0.1 and rms.max() > 10
    assert rms.max() < 1e4 and rms.min() > 1e-4
