"""Python binding of the C ABI (include/nrs.h): argument marshalling only.

torch supplies device memory and the current HIP stream; every element of
every result is computed by the HIP kernels in libnrs.so.  Names and
semantics follow the C entry points:

  rmsnorm      gamma * x / sqrt(mean(x^2) + eps) per row
  add_rmsnorm  h = round(x + residual) -> residual_out;  y = rmsnorm(h)
  mrope        in-place multimodal rotary embedding of q and k
  swiglu       silu(gate) * up over a packed [gate | up] buffer
"""
from __future__ import annotations

import ctypes

import torch

from ._native import BF16, F32, DecodeLayer, DecodeShape, check, lib

_vp = ctypes.c_void_p


def _code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"libnrs takes float32 or bfloat16 tensors, not {t.dtype}")


def _one_dtype(*ts: torch.Tensor) -> None:
    """The C ABI takes one dtype code per call: every float tensor must share it."""
    if any(t.dtype != ts[0].dtype for t in ts):
        raise TypeError("tensors of a call must share one dtype: " +
                        ", ".join(str(t.dtype) for t in ts))


def _dev(*ts: torch.Tensor) -> torch.device:
    d = ts[0].device
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError("libnrs ops take GPU tensors")
        if t.device != d:
            raise ValueError("all tensors of a call must be on one device")
    return d


try:
    _raw_stream = torch._C._cuda_getCurrentRawStream  # the current hipStream_t, no Stream object
except AttributeError:  # pragma: no cover - older torch
    _raw_stream = None


def _stream(device: torch.device) -> int:
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


class _on:
    """Make `device` current for the call; free when it already is."""

    __slots__ = ("idx", "prev")

    def __init__(self, device: torch.device):
        self.idx = device.index

    def __enter__(self):
        self.prev = torch.cuda.current_device()
        if self.prev != self.idx:
            torch.cuda.set_device(self.idx)

    def __exit__(self, *exc):
        if self.prev != self.idx:
            torch.cuda.set_device(self.prev)


def _rows2d(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dim() == 2 and t.stride(1) == 1:
        return t
    try:
        return t.view(-1, t.shape[-1])
    except RuntimeError as e:
        raise ValueError(f"{name} must be viewable as [rows, width] with unit inner stride") from e


def check_positions(pos: torch.Tensor, tokens: int, device=None) -> None:
    """pos must be int32 [3, >= tokens] with unit inner stride (temporal,
    height and width rows), on `device` when one is given.  Pure: reads only
    metadata, so it runs on CPU and meta tensors too."""
    if pos.dtype != torch.int32 or pos.dim() != 2 or pos.shape[0] != 3 or pos.stride(1) != 1:
        raise ValueError("pos must be int32 [3, >=tokens] with unit inner stride")
    if pos.shape[1] < tokens:
        raise ValueError(f"pos holds {pos.shape[1]} positions per stream, fewer than the "
                         f"{tokens} tokens")
    if device is not None and pos.device != device:
        raise ValueError("pos must be on the device of the other tensors")


def check_decode_layers(layers: list[dict], pos: torch.Tensor) -> tuple:
    """Shapes of a decode-step graph, checked before anything is recorded.

    Every layer must hold the tensors of layer 0's shapes: in_x, in_residual,
    in_y, in_residual_out [T, hidden]; in_gamma [hidden]; q [T, n_q, D];
    k [T, n_kv, D]; gate_up [T, 2 * inter]; act_out [T, inter]; and the
    post_* set either complete (same shapes as in_*) or absent.  All share one
    float dtype and device and are contiguous; pos is checked as for mrope.
    The recorded graph binds raw pointers, so a smaller tensor in any layer
    would be read or written past its end on every replay.  Returns
    (T, hidden, inter, n_q, n_kv, D).  Pure: reads only tensor metadata."""
    if not layers:
        raise ValueError("no layers")
    L0 = layers[0]
    for key in ("in_x", "q", "k", "act_out"):
        if L0.get(key) is None:
            raise ValueError(f"layer 0 has no {key}")
    if L0["in_x"].dim() != 2 or L0["q"].dim() != 3 or L0["k"].dim() != 3 or \
            L0["act_out"].dim() != 2:
        raise ValueError("in_x and act_out must be [tokens, width]; q and k [tokens, heads, D]")
    T, hidden = L0["in_x"].shape
    nq, D = L0["q"].shape[1], L0["q"].shape[2]
    nkv = L0["k"].shape[1]
    inter = L0["act_out"].shape[1]
    dtype, device = L0["in_x"].dtype, L0["in_x"].device
    if dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"libnrs takes float32 or bfloat16 tensors, not {dtype}")
    want = {"in_y": (T, hidden), "in_residual_out": (T, hidden), "in_x": (T, hidden),
            "in_residual": (T, hidden), "in_gamma": (hidden,), "q": (T, nq, D),
            "k": (T, nkv, D), "gate_up": (T, 2 * inter), "act_out": (T, inter)}
    post = {"post_y": (T, hidden), "post_residual_out": (T, hidden), "post_x": (T, hidden),
            "post_residual": (T, hidden), "post_gamma": (hidden,)}
    for i, L in enumerate(layers):
        unknown = set(L) - set(_LAYER_KEYS)
        if unknown:
            raise ValueError(f"layer {i}: unknown keys {sorted(unknown)}")
        n_post = sum(L.get(k) is not None for k in post)
        if n_post not in (0, len(post)):
            raise ValueError(f"layer {i}: the post_* tensors must be given all together or not at all")
        for key, shp in (want | (post if n_post else {})).items():
            t = L.get(key)
            if t is None:
                raise ValueError(f"layer {i} has no {key}")
            if t.dtype != dtype or t.device != device:
                raise TypeError(f"layer {i} {key}: every tensor must share in_x's dtype and device")
            if tuple(t.shape) != shp:
                raise ValueError(f"layer {i} {key}: shape {tuple(t.shape)}, expected {shp} "
                                 "(layer 0's sizes)")
            if not t.is_contiguous():
                raise ValueError(f"layer {i} {key} must be contiguous")
    check_positions(pos, T, device)
    return T, hidden, inter, nq, nkv, D


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
            out: torch.Tensor | None = None) -> torch.Tensor:
    x2 = _rows2d(x, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    y2 = _rows2d(out, "out")
    _one_dtype(x2, gamma, y2)
    d = _dev(x2, gamma, y2)
    rows, hidden = x2.shape
    if gamma.shape != (hidden,) or not gamma.is_contiguous() or y2.shape != x2.shape:
        raise ValueError("gamma must be contiguous [hidden]; out must match x")
    with _on(d):
        check(lib().nrs_rmsnorm(y2.data_ptr(), x2.data_ptr(), gamma.data_ptr(), rows, hidden,
                                x2.stride(0), y2.stride(0), float(eps), _code(x2), _stream(d)),
              "nrs_rmsnorm")
    return out


def add_rmsnorm(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
                out: torch.Tensor | None = None, residual_out: torch.Tensor | None = None):
    """Returns (y, residual_out).  Passing out=x and/or residual_out=residual
    updates in place."""
    if out is None:
        out = torch.empty_like(x)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    ts = (x, residual, out, residual_out)
    _one_dtype(*ts, gamma)
    if any(not t.is_contiguous() or t.shape != x.shape for t in ts):
        raise ValueError("x, residual, out and residual_out must be contiguous and of one shape")
    d = _dev(*ts, gamma)
    hidden = x.shape[-1]
    rows = x.numel() // hidden if hidden else 0
    if gamma.shape != (hidden,) or not gamma.is_contiguous():
        raise ValueError("gamma must be contiguous [hidden]")
    with _on(d):
        check(lib().nrs_add_rmsnorm(out.data_ptr(), residual_out.data_ptr(), x.data_ptr(),
                                    residual.data_ptr(), gamma.data_ptr(), rows, hidden, float(eps),
                                    _code(x), _stream(d)), "nrs_add_rmsnorm")
    return out, residual_out


def _beta(beta, hidden):
    if beta is not None and (beta.shape != (hidden,) or not beta.is_contiguous()):
        raise ValueError("beta must be contiguous [hidden] or None")
    return 0 if beta is None else beta.data_ptr()


def layernorm(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor | None = None,
              eps: float = 1e-5, out: torch.Tensor | None = None) -> torch.Tensor:
    """LayerNorm over the last axis; beta=None means no bias."""
    x2 = _rows2d(x, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    y2 = _rows2d(out, "out")
    _one_dtype(x2, gamma, y2, *(() if beta is None else (beta,)))
    d = _dev(x2, gamma, y2, *(() if beta is None else (beta,)))
    rows, hidden = x2.shape
    if gamma.shape != (hidden,) or not gamma.is_contiguous() or y2.shape != x2.shape:
        raise ValueError("gamma must be contiguous [hidden]; out must match x")
    b = _beta(beta, hidden)
    with _on(d):
        check(lib().nrs_layernorm(y2.data_ptr(), x2.data_ptr(), gamma.data_ptr(), b, rows, hidden,
                                  x2.stride(0), y2.stride(0), float(eps), _code(x2), _stream(d)),
              "nrs_layernorm")
    return out


def add_layernorm(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor,
                  beta: torch.Tensor | None = None, eps: float = 1e-5,
                  out: torch.Tensor | None = None, residual_out: torch.Tensor | None = None):
    """Returns (y, residual_out), y = LayerNorm(x + residual).  Passing out=x
    and/or residual_out=residual updates in place."""
    if out is None:
        out = torch.empty_like(x)
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    ts = (x, residual, out, residual_out)
    _one_dtype(*ts, gamma, *(() if beta is None else (beta,)))
    if any(not t.is_contiguous() or t.shape != x.shape for t in ts):
        raise ValueError("x, residual, out and residual_out must be contiguous and of one shape")
    d = _dev(*ts, gamma, *(() if beta is None else (beta,)))
    hidden = x.shape[-1]
    rows = x.numel() // hidden if hidden else 0
    if gamma.shape != (hidden,) or not gamma.is_contiguous():
        raise ValueError("gamma must be contiguous [hidden]")
    b = _beta(beta, hidden)
    with _on(d):
        check(lib().nrs_add_layernorm(out.data_ptr(), residual_out.data_ptr(), x.data_ptr(),
                                      residual.data_ptr(), gamma.data_ptr(), b, rows, hidden,
                                      float(eps), _code(x), _stream(d)), "nrs_add_layernorm")
    return out, residual_out


def rmsnorm_linear(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """(x / rms(x)) @ w.T over the last axis of x, with w [out_features,
    in_features] (torch's Linear layout; fold any RMSNorm gain into w)."""
    x2 = _rows2d(x, "x")
    if w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be [out_features, in_features] with unit inner stride")
    rows, n_in = x2.shape
    n_out = w.shape[0]
    if w.shape[1] != n_in:
        raise ValueError("w's in_features must match x's last dimension")
    if out is None:
        out = torch.empty(x.shape[:-1] + (n_out,), dtype=x.dtype, device=x.device)
    o2 = _rows2d(out, "out")
    if o2.shape != (rows, n_out):
        raise ValueError("out must be [rows, out_features]")
    _one_dtype(x2, w, o2)
    d = _dev(x2, w, o2)
    with _on(d):
        check(lib().nrs_rmsnorm_linear(o2.data_ptr(), x2.data_ptr(), w.data_ptr(), rows, n_in, n_out,
                                       x2.stride(0), w.stride(0), o2.stride(0), float(eps),
                                       _code(x2), _stream(d)), "nrs_rmsnorm_linear")
    return out


def mrope(q: torch.Tensor, k: torch.Tensor, pos: torch.Tensor, sections, theta: float = 1e6):
    """In place.  q: [T, n_q, D], k: [T, n_kv, D] with packed heads (token
    strides free); pos: int32 [3, >=T] with unit inner stride."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q and k must be [tokens, heads, head_dim]")
    T, nq, D = q.shape
    if k.shape[0] != T or k.shape[2] != D:
        raise ValueError("q and k disagree on tokens or head_dim")
    for t, n in ((q, "q"), (k, "k")):
        if t.shape[1] > 0 and (t.stride(2) != 1 or t.stride(1) != D):
            raise ValueError(f"{n} heads must be packed: strides (token, {D}, 1)")
    check_positions(pos, T)
    _one_dtype(q, k)
    d = _dev(q, k, pos)
    st, sh, sw = (int(s) for s in sections)
    with _on(d):
        check(lib().nrs_mrope(q.data_ptr(), k.data_ptr(), pos.data_ptr(), pos.stride(0), T, nq,
                              k.shape[1], D, q.stride(0), k.stride(0), st, sh, sw, float(theta),
                              _code(q), _stream(d)), "nrs_mrope")
    return q, k


def mrope_kv_append(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pos: torch.Tensor, sections,
                    theta: float, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    seq_idx: torch.Tensor, slot: torch.Tensor):
    """q rotated in place; rotated k and v written to k_cache / v_cache
    [n_seqs, n_kv, max_seq, D] at (seq_idx[t], slot[t]).  Returns q."""
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q: [T, n_q, D]; k, v: [T, n_kv, D]")
    T, nq, D = q.shape
    nkv = k.shape[1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.shape[1] > 0 and (t.stride(2) != 1 or t.stride(1) != D):
            raise ValueError(f"{n} heads must be packed: strides (token, {D}, 1)")
    if k_cache.shape != v_cache.shape or k_cache.dim() != 4 or k_cache.shape[1] != nkv or \
            k_cache.shape[3] != D or not k_cache.is_contiguous() or not v_cache.is_contiguous():
        raise ValueError("k_cache, v_cache must be contiguous [n_seqs, n_kv, max_seq, D]")
    for t, n in ((seq_idx, "seq_idx"), (slot, "slot")):
        if t.dtype != torch.int32 or t.shape != (T,) or not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous int32 [tokens]")
    check_positions(pos, T)
    _one_dtype(q, k, v, k_cache, v_cache)
    d = _dev(q, k, v, pos, k_cache, v_cache, seq_idx, slot)
    st, sh, sw = (int(s) for s in sections)
    with _on(d):
        check(lib().nrs_mrope_kv_append(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), pos.data_ptr(), pos.stride(0), T, nq, nkv, D,
            q.stride(0), k.stride(0), v.stride(0), st, sh, sw, float(theta), k_cache.data_ptr(),
            v_cache.data_ptr(), seq_idx.data_ptr(), slot.data_ptr(), k_cache.shape[0],
            k_cache.shape[2], _code(q), _stream(d)), "nrs_mrope_kv_append")
    return q


def swiglu(gate_up: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    gu = _rows2d(gate_up, "gate_up")
    rows, two_i = gu.shape
    if two_i % 2:
        raise ValueError("gate_up rows must have an even width [gate | up]")
    inter = two_i // 2
    if out is None:
        out = torch.empty(gate_up.shape[:-1] + (inter,), dtype=gate_up.dtype, device=gate_up.device)
    o2 = _rows2d(out, "out")
    if o2.shape != (rows, inter):
        raise ValueError("out must be [rows, inter]")
    _one_dtype(gu, o2)
    d = _dev(gu, o2)
    with _on(d):
        check(lib().nrs_swiglu(o2.data_ptr(), gu.data_ptr(), rows, inter, gu.stride(0),
                               o2.stride(0), _code(gu), _stream(d)), "nrs_swiglu")
    return out


def softmax_topk_sample(logits: torch.Tensor, temperature: float, top_k: int, u: torch.Tensor,
                        token: torch.Tensor | None = None, probs: torch.Tensor | bool = False):
    """Sample one token per row of logits [rows, vocab] from the renormalised
    top_k softmax at `temperature`, using the caller's uniforms u [rows]
    (float32).  Returns token (int32 [rows]), or (token, probs) when probs is
    True or a tensor to fill with the full softmax."""
    lg = _rows2d(logits, "logits")
    rows, vocab = lg.shape
    if u.dtype != torch.float32 or u.shape != (rows,) or not u.is_contiguous():
        raise ValueError("u must be contiguous float32 [rows]")
    if token is None:
        token = torch.empty(rows, dtype=torch.int32, device=lg.device)
    if token.dtype != torch.int32 or token.shape != (rows,) or not token.is_contiguous():
        raise ValueError("token must be contiguous int32 [rows]")
    want = probs is not False
    if probs is True:
        probs = torch.empty_like(lg)
    p2 = _rows2d(probs, "probs") if want else None
    if want and p2.shape != lg.shape:
        raise ValueError("probs must match logits")
    _one_dtype(lg, *((p2,) if want else ()))
    d = _dev(lg, u, token, *((p2,) if want else ()))
    with _on(d):
        check(lib().nrs_softmax_topk_sample(
            token.data_ptr(), p2.data_ptr() if want else None, lg.data_ptr(), rows, vocab,
            lg.stride(0), p2.stride(0) if want else 0, float(temperature), int(top_k),
            u.data_ptr(), _code(lg), _stream(d)), "nrs_softmax_topk_sample")
    return (token, probs) if want else token


class Graph:
    """A recorded hipGraph; holds references to every tensor it binds."""

    def __init__(self, handle: int, keep: list):
        self._h = handle
        self._keep = keep

    @property
    def nodes(self) -> int:
        n = lib().nrs_graph_node_count(self._h)
        if n < 0:
            check(n, "nrs_graph_node_count")
        return n

    def launch(self, stream: torch.cuda.Stream | None = None) -> None:
        s = (stream or torch.cuda.current_stream()).cuda_stream
        check(lib().nrs_graph_launch(self._h, s), "nrs_graph_launch")

    def close(self) -> None:
        if self._h:
            torch.cuda.synchronize()
            check(lib().nrs_graph_destroy(self._h), "nrs_graph_destroy")
            self._h = None
            self._keep = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_LAYER_KEYS = ("in_y", "in_residual_out", "in_x", "in_residual", "in_gamma", "q", "k", "post_y",
               "post_residual_out", "post_x", "post_residual", "post_gamma", "act_out", "gate_up")


def decode_graph(layers: list[dict], pos: torch.Tensor, sections, theta: float, eps: float) -> Graph:
    """Record the per-layer op set add_rmsnorm -> mrope -> [add_rmsnorm] ->
    swiglu of every layer into one graph.  `layers` holds, per layer, tensors
    under the nrs_decode_layer field names (post_* optional)."""
    T, hidden, inter, nq, nkv, D = check_decode_layers(layers, pos)
    L0 = layers[0]
    _dev(L0["in_x"], pos)
    keep = [pos]
    arr = (DecodeLayer * len(layers))()
    for i, L in enumerate(layers):
        for key in _LAYER_KEYS:
            t = L.get(key)
            if t is None:
                continue
            keep.append(t)
            setattr(arr[i], key, t.data_ptr())
    st, sh, sw = (int(s) for s in sections)
    shape = DecodeShape(T, hidden, inter, nq, nkv, D, pos.data_ptr(), pos.stride(0), st, sh, sw,
                        float(theta), float(eps), _code(L0["in_x"]))
    h = _vp()
    with torch.cuda.device(L0["in_x"].device):
        check(lib().nrs_decode_graph_create(ctypes.byref(h), ctypes.byref(shape), arr, len(layers)),
              "nrs_decode_graph_create")
    return Graph(h.value, keep)


def null_graph(n_nodes: int, device=None) -> Graph:
    """Calibration graph of n_nodes empty kernels."""
    h = _vp()
    with torch.cuda.device(device or torch.cuda.current_device()):
        check(lib().nrs_null_graph_create(ctypes.byref(h), int(n_nodes)), "nrs_null_graph_create")
    return Graph(h.value, [])


def stream_probe(n_read: int, n_write: int, src: list | tuple = (), dst: list | tuple = (),
                 nbytes: int | None = None, variant: int = 0, row_bytes: int = 0) -> None:
    """Measurement aid: stream n_read source and n_write destination buffers
    of nbytes bytes each (default: the first buffer's size) with the library's
    calibration kernel, pattern `variant`; row_bytes > 0 makes it a
    row-granular copy (see nrs_stream_probe in nrs.h)."""
    bufs = list(src) + list(dst)
    if len(src) != n_read or len(dst) != n_write or not bufs:
        raise ValueError("give exactly n_read sources and n_write destinations")
    if nbytes is None:
        nbytes = bufs[0].numel() * bufs[0].element_size()
    for t in bufs:
        if not t.is_contiguous() or t.numel() * t.element_size() < nbytes:
            raise ValueError("stream_probe buffers must be contiguous and hold nbytes")
    d = _dev(*bufs)
    ptr = lambda seq, i: seq[i].data_ptr() if i < len(seq) else None
    with _on(d):
        check(lib().nrs_stream_probe(ptr(dst, 0), ptr(dst, 1), ptr(src, 0), ptr(src, 1), n_read,
                                     n_write, int(nbytes), int(row_bytes), int(variant),
                                     _stream(d)),
              "nrs_stream_probe")
