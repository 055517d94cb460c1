"""Parity checks of a GPU result against the fp64 oracle (test code).

Pass bars:
  fp32 outputs: max relative error <= 1e-5 against the unrounded oracle value
    (denominator floored at FLT_MIN); for M-RoPE per rotated pair, against the
    pair norm.
  bf16 outputs: at most 1 representable step from the oracle value rounded to
    bf16 (nearest-even).  For M-RoPE an element may exceed that only where the
    rotation cancels it far below its pair's norm: there any fp32 evaluation
    carries an absolute error of a few 2^-24 of the pair norm, so the bar is
    |y - r| <= 2^-20 * |pair|; such elements are counted.
  LayerNorm: as above with the error measured against ln_scale (the size of
    the terms that make the element) in place of the element's own value; a
    bf16 element may exceed 1 step only within 2^-20 of that scale (counted).
  RMSNorm + Linear: |y - r| <= (n_in / 8 + 64) * 2^-24 * dot_scale for fp32,
    a bound on the roundings along the kernel's longest fp32 addition chain
    (steps per wave + terms per matrix-core step + waves + the scale); bf16
    outputs within 1 step of the rounded oracle value or within that bound.
  residual_out: bit-exact.
Cosine similarity is recorded for every compared tensor.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle
from numerics import FLT_MIN, bf16_steps, cosine, pair_norm, pair_rel_err, rel_err

F32_TOL = 1e-5
PAIR_ABS = 2.0**-20
REPORT = []


def check(name: str, y: torch.Tensor, r: np.ndarray, pairs: bool = False, scale=None,
          tol: float = F32_TOL, abs_frac: float = PAIR_ABS) -> dict:
    """scale: per-element error scale in place of |r| (tol applies to it for
    fp32; abs_frac * scale is the bf16 fallback bound)."""
    y = y.detach().cpu()
    yd = y.double().numpy().reshape(r.shape)
    # non-finite values pass only where the oracle holds the same one (NaN for
    # NaN, an infinity of the same sign); anywhere else they fail, whatever
    # the error metric would make of them (a NaN compares false with any bar)
    nonfinite = ~np.isfinite(yd) | ~np.isfinite(r)
    same = (yd == r) | (np.isnan(yd) & np.isnan(r))
    if (nonfinite & ~same).any():
        at = tuple(np.argwhere(nonfinite & ~same)[0])
        raise AssertionError(f"{name}: non-finite mismatch at {at}: got {yd[at]!r}, "
                             f"oracle {r[at]!r}")
    if nonfinite.any():     # matching non-finite values: compare the rest
        yd, r = np.where(nonfinite, 0.0, yd), np.where(nonfinite, 0.0, r)
        y = torch.from_numpy(np.where(nonfinite, 0.0, yd)).to(y.dtype)
    rec = {"name": name, "dtype": str(y.dtype).replace("torch.", ""), "n": int(r.size),
           "cosine": cosine(yd, r)}
    if not np.isfinite(rec["cosine"]):
        raise AssertionError(f"{name}: cosine similarity is not finite")
    if y.dtype == torch.float32:
        if scale is not None:
            err = np.abs(yd - r) / np.maximum(scale, FLT_MIN)
        else:
            err = pair_rel_err(yd, r) if pairs else rel_err(yd, r)
        worst = float(err.max()) if err.size else 0.0
        rec["max_rel_err"] = worst
        REPORT.append(rec)
        if not np.isfinite(worst) or worst > tol:
            at = np.unravel_index(int(err.argmax()), err.shape)
            raise AssertionError(f"{name}: max relative error {worst:.3e} > {tol} at {at}")
        return rec
    assert y.dtype == torch.bfloat16
    ref = oracle.round_to(r, torch.bfloat16)
    steps = bf16_steps(y, ref).reshape(r.shape)
    bad = steps > 1
    n_cancel = 0
    if pairs or scale is not None:
        ok_abs = np.abs(yd - r) <= (PAIR_ABS * pair_norm(r) if pairs else abs_frac * scale)
        n_cancel = int((bad & ok_abs).sum())
        bad &= ~ok_abs
    rec.update(max_steps=int(steps.max()) if steps.size else 0,
               over_one_step=int((steps > 1).sum()), cancellation_points=n_cancel,
               exact_frac=float((steps == 0).mean()) if steps.size else 1.0)
    REPORT.append(rec)
    if bad.any():
        at = np.argwhere(bad)[0]
        raise AssertionError(f"{name}: {int(bad.sum())} elements beyond 1 bf16 step (worst "
                             f"{int(steps.max())}), first at {tuple(at)}: got {yd[tuple(at)]!r}, "
                             f"oracle {r[tuple(at)]!r}")
    return rec


def check_exact(name: str, y: torch.Tensor, ref: torch.Tensor) -> None:
    y = y.detach().cpu()
    a = y.contiguous().view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32)
    b = ref.contiguous().view(torch.int16 if ref.dtype == torch.bfloat16 else torch.int32)
    REPORT.append({"name": name, "dtype": str(y.dtype).replace("torch.", ""), "n": y.numel(),
                   "bit_exact": bool(torch.equal(a, b))})
    if not torch.equal(a, b):
        n = int((a != b).sum())
        raise AssertionError(f"{name}: {n} elements differ from the oracle bit pattern")


def dump(path: str) -> None:
    if os.path.dirname(path):
        os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(REPORT, f, indent=1)
