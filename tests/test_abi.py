"""The C-ABI library on the CPU: it loads, exports every symbol include/nrs.h
declares, and rejects every invalid argument on the host before any HIP
call (no compute call is made here; every call below fails validation)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nrs.h")

OK, NULL, SHAPE, ALIGN, DTYPE, SECTIONS, ARG, HIP = 0, -1, -2, -3, -4, -5, -6, -7
P = 0x10000  # a 16-byte aligned stand-in address; never reaches a kernel here
U = 0x10008  # misaligned


@pytest.fixture(scope="module")
def L():
    from norm_rope_swiglu_amd import _native
    if not os.path.exists(_native.LIB_PATH):
        from norm_rope_swiglu_amd import build
        build.build()
    return _native.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nrs_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("nrs_rmsnorm", "nrs_add_rmsnorm", "nrs_mrope", "nrs_swiglu", "nrs_status_string",
              "nrs_abi_version", "nrs_decode_graph_create", "nrs_graph_launch"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    from norm_rope_swiglu_amd import _native
    out = subprocess.run(["nm", "-D", "--defined-only", _native.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(nrs_\w+)", out))
    declared = set(declared_functions())
    assert declared <= exported, declared - exported
    assert exported <= declared, f"exported but undeclared: {exported - declared}"
    assert declared == set(_native.SIGNATURES), "binding signatures differ from the header"
    for name in declared:
        assert getattr(L, name) is not None


def test_version_and_status_strings(L):
    assert L.nrs_abi_version() == 1
    for s in (OK, NULL, SHAPE, ALIGN, DTYPE, SECTIONS, ARG, HIP):
        assert L.nrs_status_string(s)
    assert L.nrs_status_string(-99) == b"unknown status"
    assert L.nrs_last_hip_error() == 0


RMS = [  # (y, x, gamma, rows, hidden, x_stride, y_stride, eps, dtype) -> status
    ((P, P, P, 4, 256, 256, 256, 1e-6, 2), DTYPE),
    ((P, P, P, -1, 256, 256, 256, 1e-6, 1), SHAPE),
    ((P, P, P, 4, 0, 256, 256, 1e-6, 1), SHAPE),
    ((P, P, P, 4, 100, 100, 100, 1e-6, 1), SHAPE),        # not a multiple of 8 bf16
    ((P, P, P, 4, 258, 258, 258, 1e-6, 0), SHAPE),        # not a multiple of 4 fp32
    ((P, P, P, 4, 65536 + 8, 65544, 65544, 1e-6, 1), SHAPE),  # wider than supported
    ((P, P, P, 4, 256, 256, 256, -1e-6, 1), ARG),
    ((P, P, P, 4, 256, 256, 256, float("nan"), 1), ARG),
    ((P, P, P, 4, 256, 256, 256, float("inf"), 1), ARG),
    ((P, P, P, 4, 256, 128, 256, 1e-6, 1), SHAPE),        # stride shorter than a row
    ((None, P, P, 4, 256, 256, 256, 1e-6, 1), NULL),
    ((P, None, P, 4, 256, 256, 256, 1e-6, 1), NULL),
    ((P, P, None, 4, 256, 256, 256, 1e-6, 1), NULL),
    ((U, P, P, 4, 256, 256, 256, 1e-6, 1), ALIGN),
    ((P, P, U, 4, 256, 256, 256, 1e-6, 1), ALIGN),
    ((P, P, P, 4, 256, 258, 256, 1e-6, 0), ALIGN),        # fp32 stride of 1032 bytes
    ((None, None, None, 0, 256, 256, 256, 1e-6, 1), OK),  # empty: nothing launched
    ((P, P, P, 1 << 31, 256, 256, 256, 1e-6, 1), SHAPE),  # more rows than 32-bit grids take
]


@pytest.mark.parametrize("args,want", RMS)
def test_rmsnorm_rejects(L, args, want):
    assert L.nrs_rmsnorm(*args, None) == want


ADD = [  # (y, residual_out, x, residual, gamma, rows, hidden, eps, dtype)
    ((P, None, P, P, P, 4, 256, 1e-6, 1), NULL),
    ((P, P, P, None, P, 4, 256, 1e-6, 1), NULL),
    ((P, U, P, P, P, 4, 256, 1e-6, 1), ALIGN),
    ((P, P, P, U, P, 4, 256, 1e-6, 1), ALIGN),
    ((P, P, P, P, P, 4, 12, 1e-6, 1), SHAPE),
    ((P, P, P, P, P, 4, 256, -1.0, 0), ARG),
    ((P, P, P, P, P, 4, 256, 1e-6, -1), DTYPE),
    ((None, None, None, None, None, 0, 256, 1e-6, 0), OK),
]


@pytest.mark.parametrize("args,want", ADD)
def test_add_rmsnorm_rejects(L, args, want):
    assert L.nrs_add_rmsnorm(*args, None) == want


LN = [  # (y, x, gamma, beta, rows, hidden, x_stride, y_stride, eps, dtype)
    ((P, P, P, P, 4, 256, 256, 256, 1e-5, 2), DTYPE),
    ((P, P, P, P, 4, 100, 100, 100, 1e-5, 1), SHAPE),
    ((P, P, P, P, 4, 256, 128, 256, 1e-5, 1), SHAPE),
    ((P, P, P, P, 4, 256, 256, 256, -1.0, 1), ARG),
    ((P, P, None, P, 4, 256, 256, 256, 1e-5, 1), NULL),
    ((P, P, P, U, 4, 256, 256, 256, 1e-5, 1), ALIGN),     # beta misaligned
    ((P, U, P, None, 4, 256, 256, 256, 1e-5, 1), ALIGN),  # no beta, x misaligned
    ((None, None, None, None, 0, 256, 256, 256, 1e-5, 1), OK),
]


@pytest.mark.parametrize("args,want", LN)
def test_layernorm_rejects(L, args, want):
    assert L.nrs_layernorm(*args, None) == want


ADD_LN = [  # (y, residual_out, x, residual, gamma, beta, rows, hidden, eps, dtype)
    ((P, None, P, P, P, P, 4, 256, 1e-5, 1), NULL),
    ((P, P, P, P, P, U, 4, 256, 1e-5, 1), ALIGN),
    ((P, P, P, U, P, None, 4, 256, 1e-5, 1), ALIGN),
    ((P, P, P, P, P, P, 4, 12, 1e-5, 1), SHAPE),
    ((P, P, P, P, P, P, 4, 256, float("nan"), 0), ARG),
    ((P, P, P, P, P, P, 4, 256, 1e-5, 7), DTYPE),
    ((None, None, None, None, None, None, 0, 256, 1e-5, 0), OK),
]


@pytest.mark.parametrize("args,want", ADD_LN)
def test_add_layernorm_rejects(L, args, want):
    assert L.nrs_add_layernorm(*args, None) == want


LIN = [  # (out, x, w, rows, n_in, n_out, x_stride, w_stride, out_stride, eps, dtype)
    ((P, P, P, 5, 2048, 4096, 2048, 2048, 4096, 1e-6, 3), DTYPE),
    ((P, P, P, -1, 2048, 4096, 2048, 2048, 4096, 1e-6, 1), SHAPE),
    ((P, P, P, 5, 0, 4096, 2048, 2048, 4096, 1e-6, 1), SHAPE),
    ((P, P, P, 5, 100, 4096, 100, 100, 4096, 1e-6, 1), SHAPE),      # not whole bf16 chunks
    ((P, P, P, 5, (1 << 20) + 8, 16, 1 << 21, 1 << 21, 16, 1e-6, 1), SHAPE),
    ((P, P, P, 5, 2048, 0, 2048, 2048, 16, 1e-6, 1), SHAPE),
    ((P, P, P, 5, 2048, 1 << 31, 2048, 2048, 1 << 31, 1e-6, 1), SHAPE),
    ((P, P, P, 5, 2048, 4096, 2040, 2048, 4096, 1e-6, 1), SHAPE),    # x stride short
    ((P, P, P, 5, 2048, 4096, 2048, 1024, 4096, 1e-6, 1), SHAPE),    # w stride short
    ((P, P, P, 5, 2048, 4096, 2048, 2048, 4000, 1e-6, 1), SHAPE),    # out stride short
    ((P, P, P, 5, 2048, 4096, 2048, 2048, 4096, -1.0, 1), ARG),
    ((P, P, P, 5, 2048, 4096, 2048, 2048, 4096, float("inf"), 0), ARG),
    ((None, P, P, 5, 2048, 4096, 2048, 2048, 4096, 1e-6, 1), NULL),
    ((P, None, P, 5, 2048, 4096, 2048, 2048, 4096, 1e-6, 1), NULL),
    ((P, P, None, 5, 2048, 4096, 2048, 2048, 4096, 1e-6, 1), NULL),
    ((P, P, U, 5, 2048, 4096, 2048, 2048, 4096, 1e-6, 1), ALIGN),
    ((P, P, P, 5, 2048, 4096, 2048, 2052, 4096, 1e-6, 1), ALIGN),    # w rows not 16-byte
    ((P + 1, P, P, 5, 2048, 4096, 2048, 2048, 4096, 1e-6, 1), ALIGN),  # out not element-aligned
    ((P + 2, P, P, 5, 2048, 4096, 2048, 2048, 4096, 1e-6, 0), ALIGN),
    ((None, None, None, 0, 2048, 4096, 2048, 2048, 4096, 1e-6, 1), OK),
    ((P, P, P, 1 << 31, 2048, 4096, 2048, 2048, 4096, 1e-6, 1), SHAPE),
]


@pytest.mark.parametrize("args,want", LIN)
def test_rmsnorm_linear_rejects(L, args, want):
    assert L.nrs_rmsnorm_linear(*args, None) == want


def test_binding_rejects_mixed_dtypes():
    import torch
    import norm_rope_swiglu_amd as nrs
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    g = torch.ones(64, dtype=torch.float32)
    for call in (lambda: nrs.rmsnorm(x, g), lambda: nrs.layernorm(x, g.bfloat16(), g),
                 lambda: nrs.add_rmsnorm(x, x, g), lambda: nrs.add_layernorm(x, x.float(), g)):
        with pytest.raises(TypeError):
            call()


def mr(q=P, k=P, pos=P, pos_stride=8, tokens=8, nq=4, nkv=2, D=64, qs=256, ks=128,
       sec=(8, 12, 12), theta=1e6, dtype=1):
    return (q, k, pos, pos_stride, tokens, nq, nkv, D, qs, ks, *sec, theta, dtype)


MROPE = [
    (mr(dtype=3), DTYPE),
    (mr(tokens=-1), SHAPE),
    (mr(nq=-1), SHAPE),
    (mr(D=0), SHAPE),
    (mr(D=72, qs=288, ks=144, sec=(12, 12, 12)), SHAPE),   # bf16 needs D % 16 == 0
    (mr(D=1024, qs=4096, ks=2048, sec=(128, 192, 192)), SHAPE),
    (mr(sec=(8, 12, 11)), SECTIONS),
    (mr(sec=(-1, 21, 12)), SECTIONS),
    (mr(theta=0.0), ARG),
    (mr(theta=float("inf")), ARG),
    (mr(theta=float("nan")), ARG),
    (mr(pos_stride=7), SHAPE),
    (mr(qs=200), SHAPE),
    (mr(ks=64), SHAPE),
    (mr(pos=None), NULL),
    (mr(q=None), NULL),
    (mr(k=None), NULL),
    (mr(pos=P + 2), ALIGN),
    (mr(q=U), ALIGN),
    (mr(qs=260), ALIGN),
    (mr(q=None, k=None, pos=None, tokens=0), OK),
    (mr(tokens=1 << 31, pos_stride=1 << 31), SHAPE),
    (mr(q=None, k=None, pos=None, nq=0, nkv=0), OK),
]


@pytest.mark.parametrize("args,want", MROPE)
def test_mrope_rejects(L, args, want):
    assert L.nrs_mrope(*args, None) == want


def kv(q=P, k=P, v=P, pos=P, pos_stride=8, tokens=8, nq=4, nkv=2, D=64, qs=256, ks=128, vs=128,
       sec=(8, 12, 12), theta=1e6, kc=P, vc=P, seq=P, slot=P, n_seqs=2, max_seq=16, dtype=1):
    return (q, k, v, pos, pos_stride, tokens, nq, nkv, D, qs, ks, vs, *sec, theta, kc, vc, seq, slot,
            n_seqs, max_seq, dtype)


KV = [
    (kv(dtype=5), DTYPE),
    (kv(sec=(8, 12, 13)), SECTIONS),
    (kv(n_seqs=0), SHAPE),
    (kv(max_seq=0), SHAPE),
    (kv(max_seq=(1 << 36) + 1), SHAPE),
    (kv(vs=64), SHAPE),
    (kv(v=None), NULL),
    (kv(kc=None), NULL),
    (kv(vc=None), NULL),
    (kv(seq=None), NULL),
    (kv(slot=None), NULL),
    (kv(v=U), ALIGN),
    (kv(kc=U), ALIGN),
    (kv(vs=132), ALIGN),
    (kv(seq=P + 1), ALIGN),
    (kv(slot=P + 2), ALIGN),
    (kv(q=None, k=None, v=None, pos=None, kc=None, vc=None, seq=None, slot=None, tokens=0), OK),
]


@pytest.mark.parametrize("args,want", KV)
def test_mrope_kv_append_rejects(L, args, want):
    assert L.nrs_mrope_kv_append(*args, None) == want


TS = [  # (token, probs, logits, rows, vocab, row_stride, probs_stride, temperature, top_k, u, dtype)
    ((P, None, P, 4, 3072, 3072, 0, 1.0, 50, P, 2), DTYPE),
    ((P, None, P, -1, 3072, 3072, 0, 1.0, 50, P, 1), SHAPE),
    ((P, None, P, 1 << 31, 3072, 3072, 0, 1.0, 50, P, 1), SHAPE),
    ((P, None, P, 4, 3070, 3070, 0, 1.0, 50, P, 1), SHAPE),       # not a multiple of 8 bf16
    ((P, None, P, 4, 3072, 3072, 0, 1.0, 0, P, 1), ARG),
    ((P, None, P, 4, 3072, 3072, 0, 1.0, 1025, P, 1), ARG),
    ((P, None, P, 4, 16, 16, 0, 1.0, 17, P, 1), ARG),             # top_k > vocab
    ((P, None, P, 4, 3072, 3072, 0, 0.0, 50, P, 1), ARG),
    ((P, None, P, 4, 3072, 3072, 0, float("inf"), 50, P, 1), ARG),
    ((P, None, P, 4, 3072, 3000, 0, 1.0, 50, P, 1), SHAPE),
    ((P, P, P, 4, 3072, 3072, 100, 1.0, 50, P, 1), SHAPE),
    ((None, None, P, 4, 3072, 3072, 0, 1.0, 50, P, 1), NULL),
    ((P, None, None, 4, 3072, 3072, 0, 1.0, 50, P, 1), NULL),
    ((P, None, P, 4, 3072, 3072, 0, 1.0, 50, None, 1), NULL),
    ((P + 2, None, P, 4, 3072, 3072, 0, 1.0, 50, P, 1), ALIGN),
    ((P, None, U, 4, 3072, 3072, 0, 1.0, 50, P, 1), ALIGN),
    ((P, None, P, 4, 3072, 3076, 0, 1.0, 50, P, 1), ALIGN),
    ((P, U, P, 4, 3072, 3072, 3072, 1.0, 50, P, 1), ALIGN),
    ((None, None, None, 0, 3072, 3072, 0, 1.0, 50, None, 1), OK),
]


@pytest.mark.parametrize("args,want", TS)
def test_softmax_topk_sample_rejects(L, args, want):
    assert L.nrs_softmax_topk_sample(*args, None) == want


SWIGLU = [  # (out, gate_up, rows, inter, gate_up_stride, out_stride, dtype)
    ((P, P, 4, 768, 1536, 768, 9), DTYPE),
    ((P, P, -2, 768, 1536, 768, 1), SHAPE),
    ((P, P, 1 << 31, 768, 1536, 768, 1), SHAPE),
    ((P, P, 4, 0, 1536, 768, 1), SHAPE),
    ((P, P, 4, 764, 1528, 764, 1), SHAPE),
    ((P, P, 4, 768, 1535, 768, 1), SHAPE),
    ((P, P, 4, 768, 1536, 767, 0), SHAPE),
    ((None, P, 4, 768, 1536, 768, 1), NULL),
    ((P, None, 4, 768, 1536, 768, 1), NULL),
    ((U, P, 4, 768, 1536, 768, 1), ALIGN),
    ((P, P, 4, 768, 1540, 768, 1), ALIGN),     # 3080-byte bf16 rows
    ((None, None, 0, 768, 1536, 768, 1), OK),
]


@pytest.mark.parametrize("args,want", SWIGLU)
def test_swiglu_rejects(L, args, want):
    assert L.nrs_swiglu(*args, None) == want


def test_graph_entry_points_reject(L):
    from norm_rope_swiglu_amd._native import DecodeLayer, DecodeShape
    h = ctypes.c_void_p()
    assert L.nrs_graph_node_count(None) == NULL
    assert L.nrs_graph_launch(None, None) == NULL
    assert L.nrs_graph_destroy(None) == OK
    assert L.nrs_null_graph_create(None, 4) == NULL
    assert L.nrs_null_graph_create(ctypes.byref(h), 0) == ARG
    shape = DecodeShape(5, 2048, 6144, 16, 8, 128, P, 5, 16, 24, 24, 1e6, 1e-6, 1)
    layers = (DecodeLayer * 1)()
    assert L.nrs_decode_graph_create(None, ctypes.byref(shape), layers, 1) == NULL
    assert L.nrs_decode_graph_create(ctypes.byref(h), None, layers, 1) == NULL
    assert L.nrs_decode_graph_create(ctypes.byref(h), ctypes.byref(shape), layers, 0) == ARG
    # layer pointers left NULL: the first op's check fails before any recording
    assert L.nrs_decode_graph_create(ctypes.byref(h), ctypes.byref(shape), layers, 1) == NULL
    bad = DecodeShape(5, 2048, 6144, 16, 8, 128, P, 5, 16, 24, 23, 1e6, 1e-6, 1)
    for f in DecodeLayer._fields_:
        setattr(layers[0], f[0], P)
    layers[0].post_x = None
    assert L.nrs_decode_graph_create(ctypes.byref(h), ctypes.byref(bad), layers, 1) == SECTIONS
    assert h.value is None


# nrs_stream_probe(dst0, dst1, src0, src1, n_read, n_write, bytes, row_bytes, variant)
STREAM = [
    ((P, None, P, None, 0, 0, 1024, 0, 0), ARG),           # nothing to move
    ((P, None, P, None, 3, 1, 1024, 0, 0), ARG),
    ((P, None, P, None, 1, 3, 1024, 0, 0), ARG),
    ((P, None, P, None, -1, 1, 1024, 0, 0), ARG),
    ((P, None, P, None, 1, 1, -16, 0, 0), SHAPE),
    ((P, None, P, None, 1, 1, 1000, 0, 0), SHAPE),         # not whole 16-byte chunks
    ((None, None, P, None, 1, 1, 1024, 0, 0), NULL),
    ((P, None, None, None, 1, 1, 1024, 0, 0), NULL),
    ((P, None, P, None, 2, 1, 1024, 0, 0), NULL),          # second source missing
    ((P, None, P, P, 2, 2, 1024, 0, 0), NULL),             # second destination missing
    ((U, None, P, None, 1, 1, 1024, 0, 0), ALIGN),
    ((P, None, U, None, 1, 1, 1024, 0, 0), ALIGN),
    ((P, P, P, U, 2, 2, 1024, 0, 0), ALIGN),
    ((None, None, None, None, 1, 1, 0, 0, 0), OK),         # empty call: no launch
    ((P, None, P, None, 1, 1, 1024, 0, 4), ARG),       # no such variant
    ((P, None, P, None, 1, 1, 1024, 0, -1), ARG),
    ((P, P, P, None, 1, 2, 4096, 1024, 0), ARG),      # row copies move as many streams each way
    ((P, None, P, P, 2, 0, 4096, 1024, 0), ARG),      # a row read takes one source
    ((P, None, None, None, 0, 1, 4096, 1024, 0), ARG),    # rows: something is read
    ((None, None, P, None, 1, 0, 4096, 1024, 2), ARG),    # row read: variants 0 and 1 only
    ((None, None, P, None, 1, 0, 4096, 1000, 0), SHAPE),  # row read: whole 16-byte chunks
    ((None, None, P, None, 1, 0, 4096, 1008, 0), SHAPE),  # row read: whole rows
    ((None, None, P, None, 1, 0, 2**31, 2**30 + 16, 0), SHAPE),  # row read: rows up to 1 GiB
    ((None, None, P, None, 1, 0, 2**31 * 32, 16, 0), SHAPE),     # row read: at most 2^31 - 1 rows
    ((None, None, None, None, 1, 0, 1008, 1008, 0), NULL),       # row read needs its source
    ((None, None, U, None, 1, 0, 1008, 1008, 0), ALIGN),
    ((P, None, P, None, 1, 1, 4096, 1024, 2), ARG),   # rows: variants 0 and 1 only
    ((P, None, P, None, 1, 1, 4096, 1000, 0), SHAPE), # rows of whole KiB
    ((P, None, P, None, 1, 1, 5120, 5120, 0), SHAPE), # 5 KiB rows are not built
    ((P, None, P, None, 1, 1, 5120, 2048, 0), SHAPE), # not a whole number of rows
    ((P, None, P, None, 1, 1, 4096, -1024, 0), SHAPE),
]


@pytest.mark.parametrize("args,want", STREAM)
def test_stream_probe_rejects(L, args, want):
    assert L.nrs_stream_probe(*args, None) == want
