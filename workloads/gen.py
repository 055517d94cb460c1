"""Counter-based seeded random numbers for the synthetic decoder-layer inputs.

This module draws numbers and nothing else: it holds none of the arithmetic of
RMSNorm, M-RoPE or SwiGLU, so both the fp64 oracle tests and the HIP path can
take their inputs from it without sharing any of the method.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014).  Output i of a stream with key K is
mix(K + (i+1)*GOLDEN); being counter-based, any element range of a tensor can
be drawn on its own, on the CPU or on a GPU, with identical integer results.
Uniforms take the top 53 bits; normals come from the Box-Muller transform
(Box and Muller, 1958) in fp64, one pair of normals per pair of counters.

Everything runs on torch int64/float64 tensors on the requested device;
uint64 arithmetic is emulated with wrapping int64 multiply and masked shifts.
"""
from __future__ import annotations

import math

import torch

GOLDEN = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
_M64 = (1 << 64) - 1

# Elements drawn per chunk: bounds the int64/float64 temporaries on a device.
_CHUNK = 1 << 25


def _as_i64(v: int) -> int:
    v &= _M64
    return v - (1 << 64) if v >= (1 << 63) else v


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of an int64 tensor viewed as uint64."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def mix64_int(z: int) -> int:
    """SplitMix64 output mix of one Python integer (used for keys and tests)."""
    z &= _M64
    z = ((z ^ (z >> 30)) * MIX1) & _M64
    z = ((z ^ (z >> 27)) * MIX2) & _M64
    return z ^ (z >> 31)


def splitmix64_int(key: int, n: int) -> list[int]:
    """First n outputs of the stream with key `key`, as Python integers."""
    return [mix64_int(key + (i + 1) * GOLDEN) for i in range(n)]


def stream_key(seed: int, name: str) -> int:
    """64-bit stream key for a named tensor: FNV-1a 64 of "seed:name", mixed."""
    h = 0xCBF29CE484222325
    for b in f"{seed}:{name}".encode():
        h = ((h ^ b) * 0x100000001B3) & _M64
    return mix64_int(h)


def raw64(key: int, start: int, n: int, device) -> torch.Tensor:
    """Outputs start..start+n-1 of stream `key` as int64 (uint64 bit patterns)."""
    ctr = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    z = ctr * _as_i64(GOLDEN) + _as_i64(key)
    z = (z ^ _srl(z, 30)) * _as_i64(MIX1)
    z = (z ^ _srl(z, 27)) * _as_i64(MIX2)
    return z ^ _srl(z, 31)


def uniform(key: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """n uniforms in [0, 1) (fp64): the top 53 bits of each output times 2^-53."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    for c0 in range(0, n, _CHUNK):
        c1 = min(n, c0 + _CHUNK)
        out[c0:c1] = _srl(raw64(key, start + c0, c1 - c0, device), 11).to(torch.float64) * 2.0**-53
    return out


def normal(key: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """n standard normals (fp64) for elements start..start+n-1 of stream `key`.

    Element e belongs to Box-Muller pair e//2, which consumes counters 2*(e//2)
    and 2*(e//2)+1: even elements take the cosine branch, odd ones the sine.
    """
    out = torch.empty(n, dtype=torch.float64, device=device)
    for c0 in range(0, n, _CHUNK):
        c1 = min(n, c0 + _CHUNK)
        e0, e1 = start + c0, start + c1
        p0, p1 = e0 // 2, (e1 + 1) // 2
        u = _srl(raw64(key, 2 * p0, 2 * (p1 - p0), device), 11).to(torch.float64) * 2.0**-53
        u1 = 1.0 - u[0::2]  # (0, 1]: log is finite
        u2 = u[1::2]
        r = torch.sqrt(-2.0 * torch.log(u1))
        ang = (2.0 * math.pi) * u2
        pair = torch.stack((r * torch.cos(ang), r * torch.sin(ang)), dim=1).reshape(-1)
        out[c0:c1] = pair[e0 - 2 * p0 : e1 - 2 * p0]
    return out


def store(v64: torch.Tensor, dtype: str) -> torch.Tensor:
    """Round fp64 draws to the storage dtype ("f32" or "bf16"), via fp32."""
    v32 = v64.to(torch.float32)
    if dtype == "f32":
        return v32
    if dtype == "bf16":
        return v32.to(torch.bfloat16)
    raise ValueError(f"unknown dtype {dtype!r}")
