"""ctypes view of the fp64 CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  Inputs are CPU torch
tensors in their storage dtype (float32 or bfloat16); results are float64
numpy arrays, unrounded, in dense row-major layout.  The arithmetic is in
oracle.c; this file only marshals pointers.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from .build import LIB, build

F32, BF16 = 0, 1
_lib = None
_i64, _int, _dbl, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("NRS_ORACLE_LIB")  # a planted-mistake build, in the mutation test
        if path is None:
            path = LIB
            if not os.path.exists(path):
                build()
        L = ctypes.CDLL(path)
        L.oracle_round.argtypes = [_vp, _vp, _i64, _int]
        L.oracle_widen.argtypes = [_vp, _vp, _i64, _int]
        L.oracle_rmsnorm.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _dbl, _int]
        L.oracle_add_rmsnorm.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _dbl, _int]
        L.oracle_layernorm.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _dbl, _int]
        L.oracle_add_layernorm.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _dbl, _int]
        L.oracle_rmsnorm_linear.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _dbl, _int]
        L.oracle_mrope.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _int, _int,
                                   _i64, _i64, _int, _int, _int, _dbl, _int]
        L.oracle_swiglu.argtypes = [_vp, _vp, _i64, _i64, _i64, _int]
        L.oracle_softmax_topk_sample.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _dbl,
                                                 _i64, _vp, _int]
        L.oracle_mrope_kv_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _int,
                                             _int, _int, _i64, _i64, _i64, _int, _int, _int, _dbl,
                                             _vp, _vp, _i64, _i64, _int]
        for f in ("oracle_round", "oracle_widen", "oracle_rmsnorm", "oracle_add_rmsnorm",
                  "oracle_mrope", "oracle_swiglu", "oracle_mrope_kv_append",
                  "oracle_softmax_topk_sample", "oracle_layernorm", "oracle_add_layernorm",
                  "oracle_rmsnorm_linear"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"oracle takes float32 or bfloat16 tensors, not {t.dtype}")


def _cpu(t: torch.Tensor) -> torch.Tensor:
    if t.device.type != "cpu":
        raise ValueError("oracle inputs must be CPU tensors")
    return t


def _ptr(a) -> int:
    return a.ctypes.data if isinstance(a, np.ndarray) else a.data_ptr()


def _f32(v: float) -> float:
    """A scalar argument as the library's C ABI receives it: rounded to fp32
    (eps and the temperature are fp32 arguments there), then widened, so the
    oracle computes with the very value the kernels use."""
    return float(np.float32(v))


def widen(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a stored fp32/bf16 tensor (any shape)."""
    t = _cpu(t).contiguous()
    out = np.empty(t.shape, dtype=np.float64)
    lib().oracle_widen(_ptr(out), _ptr(t), t.numel(), _code(t))
    return out


def round_to(r: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Round float64 values straight to fp32/bf16 (nearest, ties to even)."""
    r = np.ascontiguousarray(r, dtype=np.float64)
    out = torch.empty(r.shape, dtype=dtype)
    lib().oracle_round(_ptr(out), _ptr(r), r.size, _code(out))
    return out


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float) -> np.ndarray:
    """x: [rows, hidden] with unit column stride (rows may be strided)."""
    x = _cpu(x)
    assert x.dim() == 2 and x.stride(1) == 1 and gamma.dtype == x.dtype
    rows, hidden = x.shape
    g = _cpu(gamma).contiguous()
    y = np.empty((rows, hidden), dtype=np.float64)
    lib().oracle_rmsnorm(_ptr(y), _ptr(x), _ptr(g), rows, hidden, x.stride(0), _f32(eps), _code(x))
    return y


def add_rmsnorm(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor, eps: float):
    """Returns (y float64 [rows, hidden], residual_out tensor in x's dtype)."""
    x, residual = _cpu(x).contiguous(), _cpu(residual).contiguous()
    assert x.shape == residual.shape and x.dtype == residual.dtype == gamma.dtype
    rows, hidden = x.shape
    g = _cpu(gamma).contiguous()
    y = np.empty((rows, hidden), dtype=np.float64)
    res_out = torch.empty_like(x)
    lib().oracle_add_rmsnorm(_ptr(y), _ptr(res_out), _ptr(x), _ptr(residual), _ptr(g), rows,
                             hidden, _f32(eps), _code(x))
    return y, res_out


def layernorm(x: torch.Tensor, gamma: torch.Tensor, beta, eps: float) -> np.ndarray:
    """x: [rows, hidden] with unit column stride; beta may be None."""
    x = _cpu(x)
    assert x.dim() == 2 and x.stride(1) == 1 and gamma.dtype == x.dtype
    rows, hidden = x.shape
    g = _cpu(gamma).contiguous()
    b = None if beta is None else _cpu(beta).contiguous()
    assert b is None or b.dtype == x.dtype
    y = np.empty((rows, hidden), dtype=np.float64)
    lib().oracle_layernorm(_ptr(y), _ptr(x), _ptr(g), None if b is None else _ptr(b), rows, hidden,
                           x.stride(0), _f32(eps), _code(x))
    return y


def add_layernorm(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor, beta, eps: float):
    """Returns (y float64 [rows, hidden], residual_out tensor in x's dtype)."""
    x, residual = _cpu(x).contiguous(), _cpu(residual).contiguous()
    assert x.shape == residual.shape and x.dtype == residual.dtype == gamma.dtype
    rows, hidden = x.shape
    g = _cpu(gamma).contiguous()
    b = None if beta is None else _cpu(beta).contiguous()
    y = np.empty((rows, hidden), dtype=np.float64)
    res_out = torch.empty_like(x)
    lib().oracle_add_layernorm(_ptr(y), _ptr(res_out), _ptr(x), _ptr(residual), _ptr(g),
                               None if b is None else _ptr(b), rows, hidden, _f32(eps), _code(x))
    return y, res_out


def rmsnorm_linear(x: torch.Tensor, w: torch.Tensor, eps: float) -> np.ndarray:
    """x: [rows, n_in], w: [n_out, n_in] (unit column strides; rows may be strided)."""
    x, w = _cpu(x), _cpu(w)
    assert x.dim() == 2 and w.dim() == 2 and x.stride(1) == 1 and w.stride(1) == 1
    assert x.dtype == w.dtype and x.shape[1] == w.shape[1]
    rows, n_in = x.shape
    out = np.empty((rows, w.shape[0]), dtype=np.float64)
    lib().oracle_rmsnorm_linear(_ptr(out), _ptr(x), _ptr(w), rows, n_in, w.shape[0], x.stride(0),
                                w.stride(0), _f32(eps), _code(x))
    return out


def mrope(q: torch.Tensor, k: torch.Tensor, pos: torch.Tensor, sections, theta: float):
    """q: [T, n_q, D], k: [T, n_kv, D] (token stride free, heads packed);
    pos: int32 [3, >=T] (row stride free).  Returns (q_rot, k_rot) float64."""
    q, k, pos = _cpu(q), _cpu(k), _cpu(pos)
    assert q.dim() == 3 and k.dim() == 3 and q.dtype == k.dtype
    T, nq, D = q.shape
    nkv = k.shape[1]
    assert k.shape[0] == T and k.shape[2] == D
    assert q.stride(2) == 1 and q.stride(1) == D and k.stride(2) == 1 and k.stride(1) == D
    assert pos.dtype == torch.int32 and pos.dim() == 2 and pos.shape[0] == 3 and pos.stride(1) == 1
    assert D // 2 <= 1024
    qo = np.empty((T, nq, D), dtype=np.float64)
    ko = np.empty((T, nkv, D), dtype=np.float64)
    st, sh, sw = (int(s) for s in sections)
    lib().oracle_mrope(_ptr(qo), _ptr(ko), _ptr(q), _ptr(k), _ptr(pos), pos.stride(0), T, nq, nkv,
                       D, q.stride(0), k.stride(0), st, sh, sw, float(theta), _code(q))
    return qo, ko


def mrope_kv_append(q, k, v, pos, sections, theta, seq_idx, slot, k_cache, v_cache):
    """q: [T, n_q, D], k and v: [T, n_kv, D] (token strides free); pos int32
    [3, >=T]; seq_idx, slot int32 [T]; k_cache: float64 [n_seqs, n_kv, max_seq, D]
    (initial contents, updated copy returned); v_cache: tensor in q's dtype,
    same shape (updated copy returned).  Returns (q_rot, k_cache, v_cache)."""
    q, k, v, pos = _cpu(q), _cpu(k), _cpu(v), _cpu(pos)
    T, nq, D = q.shape
    nkv = k.shape[1]
    for t in (q, k, v):
        assert t.stride(2) == 1 and (t.shape[1] == 0 or t.stride(1) == D) and t.dtype == q.dtype
    assert v.shape == k.shape and k.shape[0] == T and k.shape[2] == D
    assert pos.dtype == torch.int32 and pos.stride(1) == 1
    seq_idx = _cpu(seq_idx).to(torch.int32).contiguous()
    slot = _cpu(slot).to(torch.int32).contiguous()
    kc = np.array(k_cache, dtype=np.float64, copy=True, order="C")
    vc = _cpu(v_cache).clone().contiguous()
    n_seqs, _, max_seq, _ = kc.shape
    assert kc.shape == (n_seqs, nkv, max_seq, D) and tuple(vc.shape) == kc.shape and vc.dtype == q.dtype
    qo = np.empty((T, nq, D), dtype=np.float64)
    st, sh, sw = (int(x) for x in sections)
    lib().oracle_mrope_kv_append(_ptr(qo), _ptr(kc), _ptr(vc), _ptr(q), _ptr(k), _ptr(v), _ptr(pos),
                                 pos.stride(0), T, nq, nkv, D, q.stride(0), k.stride(0), v.stride(0),
                                 st, sh, sw, float(theta), _ptr(seq_idx), _ptr(slot), n_seqs, max_seq,
                                 _code(q))
    return qo, kc, vc


def softmax_topk_sample(logits: torch.Tensor, temperature: float, top_k: int, u, want_probs=True):
    """logits: [rows, vocab] (row stride free); u: [rows] float32 uniforms.
    Returns (token int32 [rows], probs float64 [rows, vocab] or None,
    kept int64 [rows, top_k], cdf float64 [rows, top_k])."""
    x = _cpu(logits)
    assert x.dim() == 2 and x.stride(1) == 1
    rows, vocab = x.shape
    assert 1 <= top_k <= vocab
    uu = np.ascontiguousarray(np.asarray(u, dtype=np.float32).reshape(rows))
    tok = np.empty(rows, dtype=np.int32)
    probs = np.empty((rows, vocab), dtype=np.float64) if want_probs else None
    kept = np.empty((rows, top_k), dtype=np.int64)
    cdf = np.empty((rows, top_k), dtype=np.float64)
    lib().oracle_softmax_topk_sample(_ptr(tok), None if probs is None else _ptr(probs), _ptr(kept),
                                     _ptr(cdf), _ptr(x), rows, vocab, x.stride(0),
                                     _f32(temperature), int(top_k), _ptr(uu), _code(x))
    return tok, probs, kept, cdf


def swiglu(gate_up: torch.Tensor) -> np.ndarray:
    """gate_up: [rows, 2*inter] = [gate | up] (rows may be strided)."""
    gu = _cpu(gate_up)
    assert gu.dim() == 2 and gu.stride(1) == 1 and gu.shape[1] % 2 == 0
    rows, two_i = gu.shape
    out = np.empty((rows, two_i // 2), dtype=np.float64)
    lib().oracle_swiglu(_ptr(out), _ptr(gu), rows, two_i // 2, gu.stride(0), _code(gu))
    return out
