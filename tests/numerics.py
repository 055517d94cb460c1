"""Comparison metrics for the parity tests (test code; no op arithmetic).

fp32 outputs: relative error against the unrounded fp64 oracle value, with the
denominator floored at FLT_MIN (2^-126); for M-RoPE the error of each rotated
(j, j + D/2) pair is measured against the pair's norm, since a rotation can
cancel one component to ~0 while preserving the pair norm.

bf16 outputs: distance in representable steps between the kernel's bf16 and
the oracle value rounded to bf16 (nearest, ties to even).  Bit patterns are
mapped to monotone integers with +0 and -0 both at 0, so the step distance is
defined across binade edges and zero.

LayerNorm outputs are measured against the size of the terms that make each
element rather than the element itself: gamma * (x - mean) / sigma cancels to
~0 near the mean (and against beta), while an fp32 evaluation carries the
mean's own rounding, ~u * mean|x|, into every deviation.  ln_scale gives
|gamma| * (|x - mean| + mean|x|) / sigma + |beta| per element.

RMSNorm + Linear outputs are dot products accumulated in fp32: their error is
bounded by the number of roundings along the longest addition chain times
u = 2^-24 times sum_n |x_n / rms * w_kn| (dot_scale), whatever the output's
own size after cancellation.
"""
from __future__ import annotations

import numpy as np
import torch

FLT_MIN = 2.0**-126


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_key(bits: np.ndarray) -> np.ndarray:
    """Monotone integer of a bf16 bit pattern: -(magnitude) for negatives."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_steps(y: torch.Tensor, ref: torch.Tensor) -> np.ndarray:
    """|key(y) - key(ref)| elementwise for two bf16 tensors."""
    return np.abs(bf16_key(bf16_bits(y)) - bf16_key(bf16_bits(ref)))


def rel_err(y: np.ndarray, r: np.ndarray) -> np.ndarray:
    return np.abs(y - r) / np.maximum(np.abs(r), FLT_MIN)


def pair_rel_err(y: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Per-pair relative error for [..., D] head vectors with pairs (j, j+D/2)."""
    half = y.shape[-1] // 2
    dy = np.hypot(y[..., :half] - r[..., :half], y[..., half:] - r[..., half:])
    nr = np.hypot(r[..., :half], r[..., half:])
    return dy / np.maximum(nr, FLT_MIN)


def pair_norm(r: np.ndarray) -> np.ndarray:
    """Norm of each element's (j, j+D/2) pair, broadcast back to [..., D]."""
    half = r.shape[-1] // 2
    n = np.hypot(r[..., :half], r[..., half:])
    return np.concatenate([n, n], axis=-1)


def ln_scale(h: np.ndarray, gamma: np.ndarray, beta, eps: float) -> np.ndarray:
    """Per-element magnitude of LayerNorm's terms for rows h [rows, hidden] (fp64)."""
    mean = h.mean(axis=1, keepdims=True)
    sigma = np.sqrt(((h - mean) ** 2).mean(axis=1, keepdims=True) + eps)
    s = np.abs(gamma) * (np.abs(h - mean) + np.abs(h).mean(axis=1, keepdims=True)) / sigma
    return s if beta is None else s + np.abs(beta)


def dot_scale(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """sum_n |x[m][n] / rms_m| * |w[k][n]| for x [rows, n_in], w [n_out, n_in] (fp64)."""
    rms = np.sqrt((x * x).mean(axis=1, keepdims=True) + eps)
    return np.abs(x / rms) @ np.abs(w).T


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0.0 or nb == 0.0:
        return 1.0 if na == nb else 0.0
    return float(np.dot(a, b) / (na * nb))
