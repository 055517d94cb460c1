"""The five synthetic decoder-layer workloads, built from seeded draws.

Shapes and value distributions follow the Qwen3-TTS-1.7B-like decoder the
qwen3-tts-triton post describes (de.news.hada.io topic 27742, part 3: the four
fused ops RMSNorm, M-RoPE, Norm+Residual and SwiGLU; "5 candidates in the
time of 1" in part 1).  The pages give no tensor shapes, so the dimensions
(hidden 2048, 16 q / 8 kv heads of 128, intermediate 6144) and the position
recipes are a stated reading; every tensor is drawn here, nothing is trained.

No op arithmetic lives here: a Workload is a bag of input tensors.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

from .gen import normal, store, stream_key, uniform


@dataclass
class Layer:
    """Inputs of one decoder layer's op set (all [tokens, ...], row-major)."""

    x: torch.Tensor          # [T, H] input of the residual add (e.g. attention/MLP output)
    residual: torch.Tensor   # [T, H] residual stream
    gamma: torch.Tensor      # [H]    RMSNorm weight
    q: torch.Tensor          # [T, n_q, D]
    k: torch.Tensor          # [T, n_kv, D]
    gate_up: torch.Tensor    # [T, 2I] = [gate | up]
    x2: torch.Tensor | None = None      # [T, H] second residual input (post-attention norm)
    gamma2: torch.Tensor | None = None  # [H]    second norm weight


@dataclass
class Workload:
    name: str
    dtype: str               # "f32" or "bf16": storage and I/O type
    tokens: int
    hidden: int
    inter: int
    n_q: int
    n_kv: int
    head_dim: int
    sections: tuple[int, int, int]
    theta: float
    eps: float
    pos: torch.Tensor        # int32 [3, T]: temporal, height, width streams
    layers: list[Layer] = field(default_factory=list)
    seq_lens: list[int] | None = None

    @property
    def layer(self) -> Layer:
        return self.layers[0]


def _normal(seed, name, shape, device):
    n = math.prod(shape)
    return normal(stream_key(seed, name), n, device).reshape(shape)


def _row_scales(seed, name, rows, device):
    """Per-row scale 10^(6u-3): log-uniform in [1e-3, 1e3]."""
    u = uniform(stream_key(seed, name), rows, device)
    return torch.pow(10.0, 6.0 * u - 3.0)


def _layer(seed, cfg, li, T, H, I, nq, nkv, D, dtype, device, *, outliers=False,
           scaled=False, second_norm=False):
    tag = f"{cfg}/L{li}"
    x = _normal(seed, f"{tag}/x", (T, H), device)
    if outliers:
        # 0.5% of x entries scaled by 50 (activation outliers)
        hit = uniform(stream_key(seed, f"{tag}/x_outlier"), T * H, device).reshape(T, H) < 0.005
        x = torch.where(hit, x * 50.0, x)
    res = _normal(seed, f"{tag}/residual", (T, H), device)
    gamma = 1.0 + 0.1 * _normal(seed, f"{tag}/gamma", (H,), device)
    q = _normal(seed, f"{tag}/q", (T, nq, D), device)
    k = _normal(seed, f"{tag}/k", (T, nkv, D), device)
    gu = _normal(seed, f"{tag}/gate_up", (T, 2 * I), device)
    x2 = gamma2 = None
    if second_norm:
        x2 = _normal(seed, f"{tag}/x2", (T, H), device)
        gamma2 = 1.0 + 0.1 * _normal(seed, f"{tag}/gamma2", (H,), device)
    if scaled:
        x = x * _row_scales(seed, f"{tag}/x_scale", T, device)[:, None]
        res = res * _row_scales(seed, f"{tag}/residual_scale", T, device)[:, None]
        q = q * _row_scales(seed, f"{tag}/q_scale", T, device)[:, None, None]
        k = k * _row_scales(seed, f"{tag}/k_scale", T, device)[:, None, None]
        gu = gu * _row_scales(seed, f"{tag}/gate_up_scale", T, device)[:, None]
    s = lambda t: None if t is None else store(t, dtype).contiguous()
    return Layer(s(x), s(res), s(gamma), s(q), s(k), s(gu), s(x2), s(gamma2))


def _sections(head_dim):
    half = head_dim // 2
    # [8,12,12] of 32 pairs at head_dim 64, [16,24,24] of 64 at 128: 1/4, 3/8, 3/8
    st = half // 4
    sh = (half - st) // 2
    return (st, sh, half - st - sh)


def _same_streams(p):
    p = torch.as_tensor(p, dtype=torch.int32)
    return torch.stack((p, p, p)).contiguous()


def tiny(seed=0, device="cpu"):
    """Tiny fp32 layer: T=8, hidden 256, 4q/2kv x 64, intermediate 768."""
    T, H, I, nq, nkv, D = 8, 256, 768, 4, 2, 64
    w = Workload("tiny_f32", "f32", T, H, I, nq, nkv, D, (8, 12, 12), 1e6, 1e-6,
                 _same_streams(torch.arange(T)).to(device))
    w.layers.append(_layer(seed, "tiny", 0, T, H, I, nq, nkv, D, "f32", device))
    return w


def decode(seed=0, device="cpu", n_layers=28, second_norm=False, batch=5):
    """Decode step: `batch` sequences x 1 token, hidden 2048, q16/kv8 x 128, I 6144.

    Positions: one per sequence, 100 + floor(1401 u), identical in t/h/w.
    """
    T, H, I, nq, nkv, D = batch, 2048, 6144, 16, 8, 128
    u = uniform(stream_key(seed, "decode/pos"), T, "cpu")
    p = (100 + torch.floor(1401.0 * u)).to(torch.int64)
    w = Workload("decode_bf16", "bf16", T, H, I, nq, nkv, D, (16, 24, 24), 1e6, 1e-6,
                 _same_streams(p).to(device))
    for li in range(n_layers):
        w.layers.append(_layer(seed, "decode", li, T, H, I, nq, nkv, D, "bf16", device,
                               second_norm=second_norm))
    return w


def prefill_positions(T):
    """First 512 tokens text-like (t=h=w=n); then t constant per 64-token chunk
    (continuing the text index) and h = w cycling 0..63."""
    n = torch.arange(T, dtype=torch.int64)
    c = torch.clamp(n - 512, min=0) // 64
    r = torch.clamp(n - 512, min=0) % 64
    t = torch.where(n < 512, n, 512 + c)
    hw = torch.where(n < 512, n, r)
    return torch.stack((t, hw, hw)).to(torch.int32).contiguous()


def prefill(seed=0, device="cpu", tokens=2048):
    """Prefill: 1 sequence x 2048 tokens, decode dims, outliers in x."""
    H, I, nq, nkv, D = 2048, 6144, 16, 8, 128
    w = Workload("prefill_bf16", "bf16", tokens, H, I, nq, nkv, D, (16, 24, 24), 1e6, 1e-6,
                 prefill_positions(tokens).to(device))
    w.layers.append(_layer(seed, "prefill", 0, tokens, H, I, nq, nkv, D, "bf16", device,
                           outliers=True))
    return w


def ragged_lengths(seed=0, n_seqs=64, lo=32, hi=1024):
    u = uniform(stream_key(seed, "ragged/len"), n_seqs, "cpu")
    return [int(v) for v in (lo + torch.floor((hi - lo + 1) * u)).to(torch.int64)]


def ragged(seed=0, device="cpu", n_seqs=64, lo=32, hi=1024, hidden=2048, head_dim=128,
           inter=None):
    """Packed varlen prefill: n_seqs sequences of uniform length in [lo, hi],
    each starting at its own position offset floor(1501 u)."""
    lens = ragged_lengths(seed, n_seqs, lo, hi)
    u = uniform(stream_key(seed, "ragged/offset"), n_seqs, "cpu")
    offs = torch.floor(1501.0 * u).to(torch.int64)
    p = torch.cat([o + torch.arange(L, dtype=torch.int64) for o, L in zip(offs.tolist(), lens)])
    T = int(p.numel())
    H, D = hidden, head_dim
    nq = H // D
    nkv = nq // 2
    I = inter if inter is not None else 3 * H
    w = Workload("ragged_bf16", "bf16", T, H, I, nq, nkv, D, _sections(D), 1e6, 1e-6,
                 _same_streams(p).to(device), seq_lens=lens)
    w.layers.append(_layer(seed, "ragged", 0, T, H, I, nq, nkv, D, "bf16", device))
    return w


def sweep(seed=0, device="cpu", dtype="bf16", hidden=2048, head_dim=128, tokens=32768,
          scaled=False, eps=1e-6):
    """Width/numerics sweep: intermediate 3*hidden, n_q = hidden/head_dim,
    n_kv = n_q/2, positions t=h=w=n.  `scaled` multiplies every input row by
    10^(6u-3)."""
    H, D, T = hidden, head_dim, tokens
    nq = H // D
    nkv = nq // 2
    I = 3 * H
    name = f"sweep_{dtype}_h{H}_d{D}" + ("_scaled" if scaled else "")
    w = Workload(name, dtype, T, H, 3 * H, nq, nkv, D, _sections(D), 1e6, eps,
                 _same_streams(torch.arange(T)).to(device))
    w.layers.append(_layer(seed, name, 0, T, H, I, nq, nkv, D, dtype, device, scaled=scaled))
    return w
