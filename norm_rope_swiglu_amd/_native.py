"""ctypes loader of libnrs.so (the HIP kernels behind the C ABI of include/nrs.h).

There is no fallback: if the library is not built, or a call fails, this
raises.  Build it with `python -m norm_rope_swiglu_amd.build` (hipcc, gfx950).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnrs.so")

F32, BF16 = 0, 1
ABI_VERSION = 1

_i64, _i32, _int, _f32, _f64, _vp = (ctypes.c_int64, ctypes.c_int32, ctypes.c_int, ctypes.c_float,
                                     ctypes.c_double, ctypes.c_void_p)


class DecodeShape(ctypes.Structure):
    _fields_ = [("tokens", _i64), ("hidden", _i64), ("inter", _i64),
                ("n_q_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32),
                ("pos", _vp), ("pos_stride", _i64),
                ("sec_t", _i32), ("sec_h", _i32), ("sec_w", _i32),
                ("theta", _f64), ("eps", _f32), ("dtype", _i32)]


class DecodeLayer(ctypes.Structure):
    _fields_ = [(n, _vp) for n in (
        "in_y", "in_residual_out", "in_x", "in_residual", "in_gamma", "q", "k",
        "post_y", "post_residual_out", "post_x", "post_residual", "post_gamma",
        "act_out", "gate_up")]


class NrsError(RuntimeError):
    def __init__(self, status: int, what: str, text: str, hip_error: int):
        super().__init__(f"{what}: {text} (status {status}"
                         + (f", hipError {hip_error})" if status == -7 else ")"))
        self.status = status
        self.hip_error = hip_error


# name -> (restype, argtypes), mirroring include/nrs.h
SIGNATURES = {
    "nrs_abi_version": (_int, []),
    "nrs_status_string": (ctypes.c_char_p, [_int]),
    "nrs_last_hip_error": (_int, []),
    "nrs_rmsnorm": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _int, _vp]),
    "nrs_add_rmsnorm": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _int, _vp]),
    "nrs_rmsnorm_linear": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _f32, _int, _vp]),
    "nrs_layernorm": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _int, _vp]),
    "nrs_add_layernorm": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _int, _vp]),
    "nrs_mrope": (_int, [_vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i64, _i64,
                         _i32, _i32, _i32, _f64, _int, _vp]),
    "nrs_mrope_kv_append": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i64, _i64,
                                   _i64, _i32, _i32, _i32, _f64, _vp, _vp, _vp, _vp, _i64, _i64,
                                   _int, _vp]),
    "nrs_swiglu": (_int, [_vp, _vp, _i64, _i64, _i64, _i64, _int, _vp]),
    "nrs_softmax_topk_sample": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _i32, _vp, _int,
                                       _vp]),
    "nrs_decode_graph_create": (_int, [ctypes.POINTER(_vp), ctypes.POINTER(DecodeShape),
                                       ctypes.POINTER(DecodeLayer), _i32]),
    "nrs_null_graph_create": (_int, [ctypes.POINTER(_vp), _i32]),
    "nrs_stream_probe": (_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i32, _vp]),
    "nrs_graph_node_count": (_int, [_vp]),
    "nrs_graph_launch": (_int, [_vp, _vp]),
    "nrs_graph_destroy": (_int, [_vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m norm_rope_swiglu_amd.build`; "
                               "there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        if L.nrs_abi_version() != ABI_VERSION:
            raise RuntimeError(f"libnrs ABI {L.nrs_abi_version()} != binding ABI {ABI_VERSION}")
        _lib = L
    return _lib


def check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        raise NrsError(status, what, L.nrs_status_string(status).decode(), L.nrs_last_hip_error())
