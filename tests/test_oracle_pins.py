"""Pins of the fp64 oracle to things other than itself (CPU only).

Each op is checked against closed forms, invariants the mathematics fixes,
library routines that compute the same function another way, and hand
examples, so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one test here.
"""
from __future__ import annotations

import json
import math
import os
import zlib

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


@pytest.fixture(autouse=True)
def _rng_per_test(request):
    """Each test draws from its own generator, seeded by its id, so its inputs
    do not depend on which tests ran before it (or on which worker)."""
    global rng
    rng = np.random.default_rng(zlib.crc32(request.node.nodeid.encode()))


def t32(a):
    return torch.tensor(np.asarray(a, dtype=np.float32))


def tb16(a):
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


# ----------------------------------------------------------------- rounding

def test_round_bf16_hand_cases():
    cases = json.load(open(os.path.join(GOLDEN, "bf16_rounding.json")))["cases"]
    vals = np.array([float.fromhex(c["value"]) for c in cases])
    got = oracle.round_to(vals, torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want = np.array([int(c["bits"], 16) for c in cases], dtype=np.uint16)
    assert got.tolist() == want.tolist(), [c["why"] for c, g, w in zip(cases, got, want) if g != w]


def test_round_bf16_matches_torch_on_fp32_values():
    # For values already exact in fp32 there is one rounding, which torch's
    # fp32 -> bf16 conversion also performs (nearest, ties to even).
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    edge = np.array([2.0**-149, 2.0**-133, 2.0**-134, 3.0 * 2.0**-134, 1.17549435e-38,
                     3.3895313892515355e38, 3.3961775292304957e38, -0.0, 0.0], dtype=np.float32)
    f = np.concatenate([f, edge])
    got = oracle.round_to(f.astype(np.float64), torch.bfloat16)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_round_f32_matches_numpy():
    d = rng.standard_normal(100000) * np.exp(rng.uniform(-110, 88, 100000))
    got = oracle.round_to(d, torch.float32).numpy()
    with np.errstate(over="ignore"):          # values past fp32's range round to +-inf
        want = d.astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_widen_is_exact():
    x = torch.from_numpy(rng.standard_normal(1000).astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(oracle.widen(x), x.to(torch.float64).numpy())


# ----------------------------------------------------------------- rmsnorm

def test_rmsnorm_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "rmsnorm_hand.json")))
    y = oracle.rmsnorm(t32([g["x"]]), t32(g["gamma"]), g["eps"])[0]
    np.testing.assert_allclose(y, g["y"], rtol=1e-15)
    # the same values as closed forms
    np.testing.assert_allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-15)


@pytest.mark.parametrize("hidden", [1, 7, 256, 2048])
@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-5, 0.5])
def test_rmsnorm_matches_torch_rms_norm(hidden, eps):
    x = t32(rng.standard_normal((5, hidden)) * 3)
    gamma = t32(1 + 0.1 * rng.standard_normal(hidden))
    eps = float(np.float32(eps))
    want = torch.nn.functional.rms_norm(x.double(), (hidden,), gamma.double(), eps).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(x, gamma, eps), want, rtol=1e-13, atol=0)


def test_rmsnorm_unit_rms_at_eps0():
    x = t32(rng.standard_normal((9, 333)))
    y = oracle.rmsnorm(x, torch.ones(333), 0.0)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=1e-14)


def test_rmsnorm_constant_row_closed_form():
    c, eps, H = 0.75, 1e-2, 64
    gamma = t32(rng.uniform(0.5, 1.5, H))
    y = oracle.rmsnorm(t32(np.full((1, H), c)), gamma, eps)[0]
    eps = float(np.float32(eps))     # the fp32 eps the call carries, widened
    want = gamma.double().numpy() * c / math.sqrt(c * c + eps)
    np.testing.assert_allclose(y, want, rtol=1e-15)


def test_rmsnorm_zero_row_is_zero():
    y = oracle.rmsnorm(torch.zeros(2, 32), torch.ones(32), 1e-6)
    assert np.all(y == 0)


def test_rmsnorm_single_element():
    y = oracle.rmsnorm(t32([[-2.5]]), t32([1.5]), 0.25)[0, 0]
    assert y == pytest.approx(1.5 * -2.5 / math.sqrt(6.25 + 0.25), rel=1e-15)


def test_rmsnorm_scale_law():
    # rmsnorm_eps(a x) = rmsnorm_{eps/a^2}(x); exact invariance only at eps = 0
    x = t32(rng.standard_normal((4, 100)))
    gamma = t32(1 + 0.1 * rng.standard_normal(100))
    for a in (2.0**-10, 0.5, 8.0, 2.0**12):  # powers of two: a*x is exact in fp32
        np.testing.assert_allclose(oracle.rmsnorm(x * a, gamma, 0.0), oracle.rmsnorm(x, gamma, 0.0),
                                   rtol=1e-14)
        np.testing.assert_allclose(oracle.rmsnorm(x * a, gamma, 1e-3),
                                   oracle.rmsnorm(x, gamma, 1e-3 / a**2), rtol=1e-13)


def test_rmsnorm_symmetries():
    x = t32(rng.standard_normal((3, 50)))
    gamma = t32(1 + 0.1 * rng.standard_normal(50))
    y = oracle.rmsnorm(x, gamma, 1e-6)
    assert np.array_equal(oracle.rmsnorm(-x, gamma, 1e-6), -y)             # odd
    np.testing.assert_allclose(oracle.rmsnorm(x, gamma * 2, 1e-6), 2 * y, rtol=1e-15)  # linear in gamma
    perm = rng.permutation(50)
    np.testing.assert_allclose(oracle.rmsnorm(x[:, perm], gamma[perm], 1e-6), y[:, perm],
                               rtol=1e-14)                                     # equivariant


def test_rmsnorm_row_stride_and_bf16():
    big = tb16(rng.standard_normal((6, 96)))
    x = big[:, 16:80]                        # rows of stride 96
    gamma = tb16(1 + 0.1 * rng.standard_normal(64))
    y = oracle.rmsnorm(x, gamma, 1e-6)
    want = torch.nn.functional.rms_norm(x.double(), (64,), gamma.double(), float(np.float32(1e-6)))
    np.testing.assert_allclose(y, want.numpy(), rtol=1e-13)


# ----------------------------------------------------------------- add_rmsnorm

def test_add_rmsnorm_residual_out_f32_is_ieee_sum():
    x = rng.standard_normal((7, 300)).astype(np.float32) * np.float32(1e3)
    r = rng.standard_normal((7, 300)).astype(np.float32) * np.float32(1e-3)
    _, h = oracle.add_rmsnorm(torch.from_numpy(x), torch.from_numpy(r), torch.ones(300), 1e-6)
    assert np.array_equal(h.numpy().view(np.uint32), (x + r).view(np.uint32))


def test_add_rmsnorm_residual_out_bf16_is_rounded_sum():
    # torch adds bf16 tensors in fp32 and rounds once to bf16; fp32 holds the
    # sum of two bf16 values to within a rounding that cannot change the bf16
    # result (24 >= 2*8 + 2 bits), so both are the correctly rounded sum.
    x = tb16(rng.standard_normal((5, 512)) * 10.0 ** rng.uniform(-3, 3, (5, 512)))
    r = tb16(rng.standard_normal((5, 512)))
    _, h = oracle.add_rmsnorm(x, r, torch.ones(512, dtype=torch.bfloat16), 1e-6)
    assert torch.equal(h.view(torch.int16), (x + r).view(torch.int16))
    # hand ties: 1 + 2^-8 -> 1 ; (1 + 2^-7) + 2^-8 -> 1 + 2^-6
    _, h = oracle.add_rmsnorm(tb16([[1.0, 1.0 + 2**-7]]), tb16([[2**-8, 2**-8]]),
                              torch.ones(2, dtype=torch.bfloat16), 1e-6)
    assert h.float().tolist() == [[1.0, 1.0 + 2**-6]]


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_add_rmsnorm_equals_add_then_rmsnorm(dt):
    x = torch.from_numpy(rng.standard_normal((6, 256)).astype(np.float32)).to(dt)
    r = torch.from_numpy(rng.standard_normal((6, 256)).astype(np.float32)).to(dt)
    gamma = torch.from_numpy((1 + 0.1 * rng.standard_normal(256)).astype(np.float32)).to(dt)
    y, h = oracle.add_rmsnorm(x, r, gamma, 1e-6)
    assert np.array_equal(y, oracle.rmsnorm(h, gamma, 1e-6))


def test_add_rmsnorm_special_cases():
    r = t32(rng.standard_normal((3, 64)))
    gamma = t32(1 + 0.1 * rng.standard_normal(64))
    y, h = oracle.add_rmsnorm(-r, r, gamma, 1e-6)       # x = -residual -> h = 0 -> y = 0
    assert np.all(h.numpy() == 0) and np.all(y == 0)
    y, h = oracle.add_rmsnorm(torch.zeros_like(r), r, gamma, 1e-6)  # x = 0 -> rmsnorm(residual)
    assert torch.equal(h, r)
    np.testing.assert_allclose(y, oracle.rmsnorm(r, gamma, 1e-6), rtol=0)


# ----------------------------------------------------------------- layernorm

def test_layernorm_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "layernorm_hand.json")))
    y = oracle.layernorm(t32([g["x"]]), t32(g["gamma"]), t32(g["beta"]), g["eps"])[0]
    np.testing.assert_allclose(y, g["y"], rtol=1e-15)


@pytest.mark.parametrize("hidden", [2, 7, 256, 2048])
@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.5])
@pytest.mark.parametrize("bias", [True, False])
def test_layernorm_matches_torch_layer_norm(hidden, eps, bias):
    x = t32(rng.standard_normal((5, hidden)) * 3 + 1.5)
    gamma = t32(1 + 0.1 * rng.standard_normal(hidden))
    beta = t32(0.2 * rng.standard_normal(hidden)) if bias else None
    eps = float(np.float32(eps))
    want = torch.nn.functional.layer_norm(x.double(), (hidden,), gamma.double(),
                                          None if beta is None else beta.double(), eps).numpy()
    np.testing.assert_allclose(oracle.layernorm(x, gamma, beta, eps), want, rtol=1e-12, atol=1e-14)


def test_layernorm_zero_mean_unit_population_variance_at_eps0():
    # gamma = 1, no beta, eps = 0: every row comes out with mean 0 and variance 1
    # taken over hidden (not hidden - 1) elements
    x = t32(rng.standard_normal((9, 33)) * 4 + 7)
    y = oracle.layernorm(x, torch.ones(33), None, 0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=1e-14)


def test_layernorm_two_elements_and_constant_row():
    a, b, eps = 5.0, 2.0, 0.25
    gamma, beta = t32([1.5, -2.0]), t32([0.125, 3.0])
    y = oracle.layernorm(t32([[a, b]]), gamma, beta, eps)[0]
    r = (a - b) / 2 / math.sqrt(((a - b) / 2) ** 2 + eps)
    np.testing.assert_allclose(y, [1.5 * r + 0.125, -2.0 * -r + 3.0], rtol=1e-15)
    beta = t32(rng.standard_normal(64))
    y = oracle.layernorm(t32(np.full((2, 64), -3.25)), t32(rng.uniform(0.5, 2, 64)), beta, 1e-5)
    assert np.array_equal(y, np.broadcast_to(beta.double().numpy(), (2, 64)))  # deviations are 0


def test_layernorm_shift_and_scale_invariance():
    # multiples of 2^-10 in [-8, 8): x + c and x * 2^k are exact in fp32
    x = t32(np.round(rng.uniform(-8, 8, (4, 128)) * 1024) / 1024)
    gamma, beta = t32(1 + 0.1 * rng.standard_normal(128)), t32(rng.standard_normal(128))
    y = oracle.layernorm(x, gamma, beta, 1e-3)
    for c in (-3.0, 0.5, 16.0):
        np.testing.assert_allclose(oracle.layernorm(x + c, gamma, beta, 1e-3), y, rtol=1e-12, atol=1e-13)
    for a in (2.0**-6, 4.0, 2.0**10):   # eps scales with a^2
        np.testing.assert_allclose(oracle.layernorm(x * a, gamma, beta, 1e-3 * a * a), y, rtol=1e-12,
                                   atol=1e-13)


def test_layernorm_of_zero_mean_row_is_rmsnorm_plus_beta():
    x = rng.standard_normal((3, 64))
    x = np.concatenate([x, -x], axis=1)              # every row sums to exactly 0
    x, gamma = t32(x), t32(1 + 0.1 * rng.standard_normal(128))
    beta = t32(rng.standard_normal(128))
    np.testing.assert_allclose(oracle.layernorm(x, gamma, beta, 1e-6),
                               oracle.rmsnorm(x, gamma, 1e-6) + beta.double().numpy(), rtol=1e-13, atol=1e-15)


def test_layernorm_row_stride_and_bf16():
    big = tb16(rng.standard_normal((6, 96)) + 2)
    x = big[:, 16:80]
    gamma, beta = tb16(1 + 0.1 * rng.standard_normal(64)), tb16(rng.standard_normal(64))
    y = oracle.layernorm(x, gamma, beta, 1e-5)
    want = torch.nn.functional.layer_norm(x.double(), (64,), gamma.double(), beta.double(),
                                          float(np.float32(1e-5)))
    np.testing.assert_allclose(y, want.numpy(), rtol=1e-12, atol=1e-12)   # y ~ 1: torch rounds differently


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_add_layernorm_is_rounded_sum_then_layernorm(dt):
    x = torch.from_numpy(rng.standard_normal((6, 256)).astype(np.float32) * 10).to(dt)
    r = torch.from_numpy(rng.standard_normal((6, 256)).astype(np.float32)).to(dt)
    gamma = torch.from_numpy((1 + 0.1 * rng.standard_normal(256)).astype(np.float32)).to(dt)
    beta = torch.from_numpy(rng.standard_normal(256).astype(np.float32)).to(dt)
    y, h = oracle.add_layernorm(x, r, gamma, beta, 1e-5)
    assert torch.equal(h.view(torch.int16) if dt == torch.bfloat16 else h, (x + r).view(torch.int16)
                       if dt == torch.bfloat16 else x + r)
    want = torch.nn.functional.layer_norm((x + r).double(), (256,), gamma.double(), beta.double(),
                                          float(np.float32(1e-5)))
    np.testing.assert_allclose(y, want.numpy(), rtol=1e-12, atol=1e-14)
    y0, _ = oracle.add_layernorm(x, r, gamma, None, 1e-5)
    np.testing.assert_allclose(y - y0, np.broadcast_to(beta.double().numpy(), y.shape), rtol=1e-12,
                               atol=1e-13)


# ----------------------------------------------------------------- rmsnorm + linear

def test_rmsnorm_linear_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "rmsnorm_linear_hand.json")))
    out = oracle.rmsnorm_linear(t32(g["x"]), t32(g["w"]), g["eps"])
    np.testing.assert_allclose(out, g["out"], rtol=1e-15, atol=0)


@pytest.mark.parametrize("n_in,n_out", [(8, 3), (64, 200), (256, 96)])
@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.25])
def test_rmsnorm_linear_is_rmsnorm_then_matmul(n_in, n_out, eps):
    # the pinned RMSNorm (gain 1) followed by numpy's matmul with w transposed
    x = t32(rng.standard_normal((7, n_in)) * 2)
    w = t32(rng.standard_normal((n_out, n_in)) / math.sqrt(n_in))
    eps = float(np.float32(eps))
    want = oracle.rmsnorm(x, torch.ones(n_in), eps) @ w.double().numpy().T
    np.testing.assert_allclose(oracle.rmsnorm_linear(x, w, eps), want, rtol=1e-12, atol=1e-13)


def test_rmsnorm_linear_gain_folds_into_weight_columns():
    x = t32(rng.standard_normal((4, 48)))
    gamma = t32(1 + 0.2 * rng.standard_normal(48))
    w = t32(rng.standard_normal((20, 48)))
    folded = t32(w.double().numpy() * gamma.double().numpy()[None, :])
    want = oracle.rmsnorm(x, gamma, 1e-6) @ w.double().numpy().T
    np.testing.assert_allclose(oracle.rmsnorm_linear(x, folded, 1e-6), want, rtol=1e-6, atol=1e-6)


def test_rmsnorm_linear_identity_weight_and_invariances():
    x = t32(rng.standard_normal((5, 32)))
    eye = torch.eye(32)
    np.testing.assert_allclose(oracle.rmsnorm_linear(x, eye, 1e-6),
                               oracle.rmsnorm(x, torch.ones(32), 1e-6), rtol=1e-14, atol=0)
    w = t32(rng.standard_normal((9, 32)))
    base = oracle.rmsnorm_linear(x, w, 0.0)
    for a in (2.0**-5, 8.0):                         # scale-free at eps = 0
        np.testing.assert_allclose(oracle.rmsnorm_linear(x * a, w, 0.0), base, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(oracle.rmsnorm_linear(x, w * 4, 0.0), 4 * base, rtol=1e-14, atol=0)
    np.testing.assert_allclose(oracle.rmsnorm_linear(x, w[[3, 0, 8]], 0.0), base[:, [3, 0, 8]], rtol=0)


def test_rmsnorm_linear_strides_and_bf16():
    xb = tb16(rng.standard_normal((6, 100)))
    wb = tb16(rng.standard_normal((40, 90)) * 0.1)
    x, w = xb[:, 10:74], wb[3:37, 20:84]             # strided rows of both operands
    out = oracle.rmsnorm_linear(x, w, 1e-5)
    want = torch.nn.functional.rms_norm(x.double(), (64,), None, float(np.float32(1e-5))) @ w.double().T
    np.testing.assert_allclose(out, want.numpy(), rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------- mrope

def _pos(t, h, w):
    return torch.tensor(np.array([t, h, w]), dtype=torch.int32)


def test_mrope_hand_example():
    # head_dim 4: pairs (0, 2) and (1, 3); sections [1, 1, 0]; theta 1e4.
    # pair 0 follows the temporal stream with frequency theta^0 = 1,
    # pair 1 the height stream with frequency theta^(-2/4) = 0.01.
    q = t32([[[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 1.0]]])   # [T=1, heads=2, D=4]
    k = t32([[[0.0, 0.0, 2.0, 0.0]]])
    pos = _pos([1], [2], [5])
    qo, ko = oracle.mrope(q, k, pos, (1, 1, 0), 1e4)
    c1, s1 = math.cos(1.0), math.sin(1.0)
    c2, s2 = math.cos(0.02), math.sin(0.02)
    np.testing.assert_allclose(qo[0, 0], [c1, 0.0, s1, 0.0], rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(qo[0, 1], [0.0, c2 - s2, 0.0, s2 + c2], rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(ko[0, 0], [-2 * s1, 0.0, 2 * c1, 0.0], rtol=1e-15, atol=1e-16)


def _rand_qk(T, nq, nkv, D, dt=torch.float32):
    q = torch.from_numpy(rng.standard_normal((T, nq, D)).astype(np.float32)).to(dt)
    k = torch.from_numpy(rng.standard_normal((T, nkv, D)).astype(np.float32)).to(dt)
    return q, k


@pytest.mark.parametrize("D,sections", [(64, (8, 12, 12)), (128, (16, 24, 24)), (2, (1, 0, 0))])
def test_mrope_equal_streams_is_complex_rope(D, sections):
    # Three equal streams reduce M-RoPE to plain RoPE: multiply the complex
    # number v_j + i v_(j+D/2) by exp(i p theta^(-2j/D)) (numpy complex exp).
    T, theta = 11, 1e6
    q, k = _rand_qk(T, 4, 2, D)
    p = rng.integers(0, 40000, T)
    qo, ko = oracle.mrope(q, k, _pos(p, p, p), sections, theta)
    half = D // 2
    freq = theta ** (-2.0 * np.arange(half) / D)
    rot = np.exp(1j * p[:, None, None] * freq[None, None, :])
    for v, out in ((q, qo), (k, ko)):
        z = v.double().numpy()
        zc = (z[..., :half] + 1j * z[..., half:]) * rot
        # two fp64 evaluations of the angle p * theta^(-2j/D) (C pow vs numpy's)
        # may differ by a few ulps of p: the rotated pair then moves by up to
        # |pair| * p * 2^-52 * a few
        tol = 8 * 2.0**-52 * float(p.max()) * float(np.abs(z).max()) * math.sqrt(2) + 1e-15
        np.testing.assert_allclose(out[..., :half], zc.real, rtol=0, atol=tol)
        np.testing.assert_allclose(out[..., half:], zc.imag, rtol=0, atol=tol)


def test_mrope_frequency_schedule():
    # Unit vectors in pair j at position 1 turn by the pair's frequency:
    # pair 0 by exactly 1 rad, and consecutive pairs by a constant ratio theta^(-2/D).
    D, theta = 16, 1e4
    q = torch.zeros(1, D // 2, D)
    for j in range(D // 2):
        q[0, j, j] = 1.0
    qo, _ = oracle.mrope(q, torch.zeros(1, 1, D), _pos([1], [1], [1]), (2, 3, 3), theta)
    ang = np.array([math.atan2(qo[0, j, j + D // 2], qo[0, j, j]) for j in range(D // 2)])
    assert ang[0] == pytest.approx(1.0, rel=1e-15)
    np.testing.assert_allclose(ang[1:] / ang[:-1], theta ** (-2.0 / D), rtol=1e-13)


def test_mrope_preserves_pair_norms_and_identity_at_zero():
    q, k = _rand_qk(7, 3, 1, 64)
    p = rng.integers(0, 5000, (3, 7))
    qo, ko = oracle.mrope(q, k, torch.tensor(p, dtype=torch.int32), (8, 12, 12), 1e6)
    for v, out in ((q, qo), (k, ko)):
        z = v.double().numpy()
        np.testing.assert_allclose(np.hypot(out[..., :32], out[..., 32:]),
                                   np.hypot(z[..., :32], z[..., 32:]), rtol=1e-14)
    zero = torch.zeros(3, 7, dtype=torch.int32)
    qo, ko = oracle.mrope(q, k, zero, (8, 12, 12), 1e6)
    assert np.array_equal(qo, q.double().numpy()) and np.array_equal(ko, k.double().numpy())


def test_mrope_relative_position():
    # <R(p) q, R(p') k> depends only on p - p' (each stream shifted alike).
    D = 64
    q, k = _rand_qk(1, 1, 1, D)
    def dot(pq, pk):
        qo, _ = oracle.mrope(q, k, _pos([pq[0]], [pq[1]], [pq[2]]), (8, 12, 12), 1e6)
        _, ko = oracle.mrope(q, k, _pos([pk[0]], [pk[1]], [pk[2]]), (8, 12, 12), 1e6)
        return float(np.dot(qo[0, 0], ko[0, 0]))
    base = dot((10, 20, 30), (3, 5, 7))
    for c in (1, 100, 2000):
        assert dot((10 + c, 20 + c, 30 + c), (3 + c, 5 + c, 7 + c)) == pytest.approx(base, abs=1e-11)
    assert abs(dot((10, 20, 31), (3, 5, 7)) - base) > 1e-6   # a change in one stream matters


def test_mrope_composition_and_inverse():
    q, k = _rand_qk(5, 2, 2, 32)
    p1 = rng.integers(-3000, 3000, (3, 5))
    p2 = rng.integers(-3000, 3000, (3, 5))
    P = lambda a: torch.tensor(a, dtype=torch.int32)
    a_q, a_k = oracle.mrope(q, k, P(p1), (4, 6, 6), 1e6)
    b_q, b_k = oracle.mrope(t32(a_q), t32(a_k), P(p2), (4, 6, 6), 1e6)  # via fp32 storage
    c_q, c_k = oracle.mrope(q, k, P(p1 + p2), (4, 6, 6), 1e6)
    np.testing.assert_allclose(b_q, c_q, atol=1e-6)
    np.testing.assert_allclose(b_k, c_k, atol=1e-6)
    i_q, _ = oracle.mrope(t32(a_q), t32(a_k), P(-p1), (4, 6, 6), 1e6)
    np.testing.assert_allclose(i_q, q.double().numpy(), atol=1e-6)


def test_mrope_sections_select_streams():
    D, sec = 64, (8, 12, 12)
    q, k = _rand_qk(4, 2, 1, D)
    p = rng.integers(0, 1000, (3, 4))
    base, _ = oracle.mrope(q, k, torch.tensor(p, dtype=torch.int32), sec, 1e6)
    bounds = [(0, 8), (8, 20), (20, 32)]
    for s, (lo, hi) in enumerate(bounds):
        p2 = p.copy()
        p2[s, 2] += 17                        # move stream s of token 2 only
        out, _ = oracle.mrope(q, k, torch.tensor(p2, dtype=torch.int32), sec, 1e6)
        changed = np.any(out != base, axis=1)  # [T, D]
        mask = np.zeros(D, bool)
        mask[lo:hi] = mask[32 + lo:32 + hi] = True
        assert np.all(changed[2] == mask)
        assert not changed[[0, 1, 3]].any()
    # all pairs on the temporal stream: height and width are ignored
    p3 = p.copy()
    p3[1:] += 999
    a, _ = oracle.mrope(q, k, torch.tensor(p, dtype=torch.int32), (32, 0, 0), 1e6)
    b, _ = oracle.mrope(q, k, torch.tensor(p3, dtype=torch.int32), (32, 0, 0), 1e6)
    assert np.array_equal(a, b)


def test_mrope_token_stride_and_bf16():
    T, nq, nkv, D = 6, 4, 2, 64
    qkv = tb16(rng.standard_normal((T, (nq + 2 * nkv) * D)))
    q = qkv[:, : nq * D].view(T, nq, D)
    k = qkv[:, nq * D : (nq + nkv) * D].view(T, nkv, D)
    p = torch.tensor(rng.integers(0, 3000, (3, T)), dtype=torch.int32)
    a_q, a_k = oracle.mrope(q, k, p, (8, 12, 12), 1e6)
    b_q, b_k = oracle.mrope(q.contiguous(), k.contiguous(), p, (8, 12, 12), 1e6)
    assert np.array_equal(a_q, b_q) and np.array_equal(a_k, b_k)
    # positions read with their own row stride
    wide = torch.zeros(3, 10, dtype=torch.int32)
    wide[:, :T] = p
    c_q, _ = oracle.mrope(q, k, wide[:, :T], (8, 12, 12), 1e6)
    assert np.array_equal(a_q, c_q)


# ----------------------------------------------------------------- swiglu

def _gu(gate, up):
    return t32(np.concatenate([np.atleast_2d(gate), np.atleast_2d(up)], axis=1))


def test_swiglu_closed_forms():
    g = np.array([0.0, 1.0, -1.0, 2.5, -89.0, -1000.0, 30.0])
    out = oracle.swiglu(_gu(g, np.ones_like(g)))[0]
    g32 = g.astype(np.float32).astype(np.float64)
    assert out[0] == 0.0                                   # silu(0) = 0
    assert out[1] == pytest.approx(1 / (1 + math.exp(-1)), rel=1e-15)
    assert out[2] == pytest.approx(-1 / (1 + math.e), rel=1e-15)
    assert out[3] == pytest.approx(2.5 / (1 + math.exp(-2.5)), rel=1e-15)
    assert out[4] == pytest.approx(-89 * math.exp(-89) / (1 + math.exp(-89)), rel=1e-14)
    assert out[5] == 0.0 or abs(out[5]) < 1e-300          # silu -> 0 as g -> -inf
    assert abs(out[6] - 30.0) <= 30.0 * math.exp(-30.0)    # silu(x) -> x
    del g32


def test_swiglu_odd_part_identity_and_tanh_form():
    # silu(x) - silu(-x) = x, and sigmoid(x) = (1 + tanh(x/2)) / 2
    g = (rng.standard_normal(500) * 8).astype(np.float32).astype(np.float64)
    out = oracle.swiglu(_gu(np.concatenate([g, -g]), np.ones(1000)))[0]
    np.testing.assert_allclose(out[:500] - out[500:], g, rtol=1e-14, atol=1e-300)
    # 1 + tanh(g/2) cancels for very negative g: compare where it is well conditioned
    ok = g > -6.0
    tanh_form = g * 0.5 * (1.0 + np.tanh(g / 2.0))
    np.testing.assert_allclose(out[:500][ok], tanh_form[ok], rtol=1e-12, atol=1e-300)


def test_swiglu_matches_torch_silu():
    gu = t32(rng.standard_normal((9, 2 * 321)) * 4)
    want = (torch.nn.functional.silu(gu[:, :321].double()) * gu[:, 321:].double()).numpy()
    np.testing.assert_allclose(oracle.swiglu(gu), want, rtol=1e-14)


def test_swiglu_gate_is_first_half_and_row_stride():
    out = oracle.swiglu(_gu([100.0], [2.0]))[0, 0]
    assert out == pytest.approx(200.0, rel=1e-15)       # silu(100) * 2, not silu(2) * 100
    big = tb16(rng.standard_normal((5, 200)))
    a = oracle.swiglu(big[:, 20:180])                     # inter 80, rows of stride 200
    b = oracle.swiglu(big[:, 20:180].contiguous())
    assert np.array_equal(a, b)


def test_swiglu_large_negative_gate_keeps_tiny_values():
    # silu(-95) * 1e3 ~ -5e-37 is a normal fp32 value; a formula whose exp
    # overflows would return 0 here.
    out = oracle.swiglu(_gu([-95.0, -120.0], [1e3, 1e30]))[0]
    assert out[0] == pytest.approx(-95 * math.exp(-95) * 1e3, rel=1e-14)
    assert out[1] == pytest.approx(-120 * math.exp(-120) * float(np.float32(1e30)), rel=1e-14)


# ----------------------------------------------------------------- mrope + KV-cache append

def _kv_case(dt=torch.float32, T=5, nq=2, nkv=2, D=8, n_seqs=3, max_seq=4):
    q, k = _rand_qk(T, nq, nkv, D, dt)
    v = torch.from_numpy(rng.standard_normal((T, nkv, D)).astype(np.float32)).to(dt)
    kc = np.full((n_seqs, nkv, max_seq, D), -7.0)
    vc = torch.full((n_seqs, nkv, max_seq, D), -3.0).to(dt)
    return q, k, v, kc, vc


def test_kv_append_placement_by_hand():
    # positions 0: the rotation is the identity, so the cache must hold k and
    # v themselves at [seq][head][slot][:]
    q, k, v, kc, vc = _kv_case()
    seq = torch.tensor([2, 0, 1, 0, 2], dtype=torch.int32)
    slot = torch.tensor([3, 0, 1, 2, 0], dtype=torch.int32)
    pos = torch.zeros(3, 5, dtype=torch.int32)
    qo, kc2, vc2 = oracle.mrope_kv_append(q, k, v, pos, (1, 1, 2), 1e4, seq, slot, kc, vc)
    for t, (b, s_) in enumerate(zip(seq.tolist(), slot.tolist())):
        for h in range(2):
            assert np.array_equal(kc2[b, h, s_], k[t, h].double().numpy())
            assert torch.equal(vc2[b, h, s_], v[t, h])
    written = {(b, s_) for b, s_ in zip(seq.tolist(), slot.tolist())}
    for b in range(3):
        for s_ in range(4):
            if (b, s_) not in written:
                assert np.all(kc2[b, :, s_] == -7.0) and torch.all(vc2[b, :, s_] == -3.0)
    assert np.array_equal(qo, q.double().numpy())


def test_kv_append_rotates_like_mrope_and_skips_out_of_range():
    for dt in (torch.float32, torch.bfloat16):
        q, k, v, kc, vc = _kv_case(dt, T=6, nq=3, nkv=2, D=16, n_seqs=2, max_seq=5)
        seq = torch.tensor([0, 1, 1, 2, 0, -1], dtype=torch.int32)     # 2 and -1: no such sequence
        slot = torch.tensor([4, 0, 5, 1, -1, 2], dtype=torch.int32)    # 5 and -1: no such slot
        pos = torch.tensor(rng.integers(0, 3000, (3, 6)), dtype=torch.int32)
        qo, kc2, vc2 = oracle.mrope_kv_append(q, k, v, pos, (2, 3, 3), 1e6, seq, slot, kc, vc)
        rq, rk = oracle.mrope(q, k, pos, (2, 3, 3), 1e6)
        assert np.array_equal(qo, rq)
        assert np.array_equal(kc2[0, :, 4], rk[0]) and np.array_equal(kc2[1, :, 0], rk[1])
        assert torch.equal(vc2[0, :, 4], v[0]) and torch.equal(vc2[1, :, 0], v[1])
        untouched = np.ones((2, 5), bool)
        untouched[0, 4] = untouched[1, 0] = False
        for b in range(2):
            for s_ in range(5):
                if untouched[b, s_]:
                    assert np.all(kc2[b, :, s_] == -7.0)
                    assert torch.all(vc2[b, :, s_] == torch.tensor(-3.0).to(dt))


# ----------------------------------------------------------------- softmax + top-k sampling

def _sample(logits, T, k, u, dt=torch.float32):
    x = torch.tensor(np.atleast_2d(np.asarray(logits, dtype=np.float32))).to(dt)
    return oracle.softmax_topk_sample(x, T, k, np.atleast_1d(np.asarray(u, dtype=np.float32)))


def test_topk_sample_closed_form():
    # logits 0..3, T = 1, k = 2: kept (3, 2) with probabilities e^3 : e^2, so
    # the first cumulative probability is e/(e+1) = sigmoid(1)
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    tok, probs, kept, cdf = _sample([0, 1, 2, 3], 1.0, 2, 0.7)
    assert kept[0].tolist() == [3, 2] and tok[0] == 3
    assert cdf[0, 0] == pytest.approx(s1, rel=1e-15) and cdf[0, 1] == pytest.approx(1.0, rel=1e-15)
    assert _sample([0, 1, 2, 3], 1.0, 2, 0.75)[0][0] == 2
    e = np.exp(np.arange(4.0))
    np.testing.assert_allclose(probs[0], e / e.sum(), rtol=1e-15)
    # temperature 2 halves the logits: 0 and 2 -> sigmoid(1) again
    tok, _, kept, cdf = _sample([0, 2], 2.0, 2, 0.7)
    assert kept[0].tolist() == [1, 0] and tok[0] == 1
    assert cdf[0, 0] == pytest.approx(s1, rel=1e-15)


def test_topk_sample_ties_and_boundaries():
    tok, _, kept, _ = _sample([1, 5, 5, 5, 0], 1.0, 2, 0.1)
    assert kept[0].tolist() == [1, 2]                  # equal logits: lower index first
    # u exactly at a cumulative probability: the next token (strictly greater)
    tok, _, kept, cdf = _sample([0, 0], 1.0, 2, 0.5)
    assert cdf[0, 0] == 0.5 and tok[0] == 1
    assert _sample([0, 0], 1.0, 2, 0.4999)[0][0] == 0
    # k = 1 is greedy whatever u is; u near 1 takes the last kept token
    for u in (0.0, 0.3, 0.999999):
        assert _sample([0.5, 3.0, -1.0, 3.0], 0.7, 1, u)[0][0] == 1
    assert _sample([0, 1, 2, 3], 1.0, 3, 0.9999999)[0][0] == 1


@pytest.mark.parametrize("T", [0.5, 1.0, 1.7])
def test_topk_sample_matches_torch_softmax_and_topk(T):
    x = torch.from_numpy(rng.standard_normal((4, 3000)).astype(np.float32) * 4)
    tok, probs, kept, cdf = oracle.softmax_topk_sample(x, T, 50, rng.random(4).astype(np.float32))
    T32 = float(np.float32(T))       # the fp32 temperature the call carries, widened
    np.testing.assert_allclose(probs, torch.softmax(x.double() / T32, dim=1).numpy(), rtol=1e-12)
    tk = torch.topk(x.double(), 50, dim=1, sorted=True).indices.numpy()
    assert np.array_equal(kept, tk)
    ren = np.take_along_axis(probs, kept, axis=1)
    np.testing.assert_allclose(cdf, np.cumsum(ren / ren.sum(axis=1, keepdims=True), axis=1), rtol=1e-12)


def test_topk_sample_inverse_cdf_frequencies():
    # stratified uniforms (i + 1/2)/N: token j must be drawn N * p_j +- 1 times
    x = torch.from_numpy(rng.standard_normal(64).astype(np.float32) * 2)
    N = 20000
    u = (np.arange(N) + 0.5) / N
    tok, probs, _, _ = oracle.softmax_topk_sample(x.repeat(N, 1), 1.0, 64, u.astype(np.float32))
    counts = np.bincount(tok, minlength=64)
    assert np.all(np.abs(counts - N * probs[0]) <= 1.5)
