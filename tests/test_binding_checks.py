"""The binding's shape checks (CPU, on meta tensors: no memory, no GPU).

A recorded decode graph binds raw pointers and the C ABI sees only the sizes
of layer 0, so the binding must refuse any layer whose tensors differ from
layer 0's shapes, and positions that are not int32 [3, >= tokens] with unit
inner stride, before anything is recorded or launched.
"""
from __future__ import annotations

import pytest
import torch

from norm_rope_swiglu_amd.ops import check_decode_layers, check_positions

T, H, I, NQ, NKV, D = 5, 2048, 6144, 16, 8, 128
META = torch.device("meta")


def _t(*shape, dtype=torch.bfloat16):
    return torch.empty(*shape, dtype=dtype, device=META)


def _layer(post=False, **over):
    L = {"in_x": _t(T, H), "in_residual": _t(T, H), "in_y": _t(T, H), "in_residual_out": _t(T, H),
         "in_gamma": _t(H), "q": _t(T, NQ, D), "k": _t(T, NKV, D), "gate_up": _t(T, 2 * I),
         "act_out": _t(T, I)}
    if post:
        L.update(post_x=_t(T, H), post_residual=_t(T, H), post_y=_t(T, H),
                 post_residual_out=_t(T, H), post_gamma=_t(H))
    L.update(over)
    return L


def _pos(n=T, dtype=torch.int32):
    return torch.empty(3, n, dtype=dtype, device=META)


@pytest.mark.parametrize("post", [False, True])
def test_consistent_layers_pass(post):
    assert check_decode_layers([_layer(post) for _ in range(28)], _pos()) == (T, H, I, NQ, NKV, D)


def test_longer_positions_pass():
    check_decode_layers([_layer()], _pos(T + 7))


@pytest.mark.parametrize("key,shape", [
    ("gate_up", (T, 2 * I - 8)), ("act_out", (T, I // 2)), ("q", (T, NQ // 2, D)),
    ("k", (T, NKV, D // 2)), ("in_x", (T - 1, H)), ("in_residual", (T, H // 2)),
    ("in_y", (T, H - 8)), ("in_residual_out", (T + 1, H)), ("in_gamma", (H // 2,)),
    ("q", (T, NQ * D)),
])
def test_a_smaller_or_reshaped_later_layer_is_refused(key, shape):
    layers = [_layer(), _layer(), _layer(**{key: _t(*shape)})]
    with pytest.raises(ValueError, match="layer 2"):
        check_decode_layers(layers, _pos())


def test_a_wrong_post_tensor_is_refused():
    layers = [_layer(True), _layer(True, post_gamma=_t(H // 2))]
    with pytest.raises(ValueError, match="post_gamma"):
        check_decode_layers(layers, _pos())


def test_a_partial_post_set_is_refused():
    L = _layer(True)
    del L["post_residual"]
    with pytest.raises(ValueError, match="all together"):
        check_decode_layers([_layer(True), L], _pos())


def test_a_missing_tensor_is_refused():
    L = _layer()
    del L["gate_up"]
    with pytest.raises(ValueError, match="gate_up"):
        check_decode_layers([_layer(), L], _pos())


def test_unknown_keys_are_refused():
    with pytest.raises(ValueError, match="unknown"):
        check_decode_layers([_layer(gate=_t(T, I))], _pos())


def test_dtype_mismatch_is_refused():
    with pytest.raises(TypeError):
        check_decode_layers([_layer(), _layer(k=_t(T, NKV, D, dtype=torch.float32))], _pos())


def test_non_contiguous_is_refused():
    big = _t(T, 2 * H)
    with pytest.raises(ValueError, match="contiguous"):
        check_decode_layers([_layer(), _layer(in_x=big[:, :H])], _pos())


@pytest.mark.parametrize("pos", [
    _pos(dtype=torch.int64),                      # would be read as pairs of int32
    _pos(T - 1),                                  # fewer positions than tokens
    torch.empty(2, T, dtype=torch.int32, device=META),
    torch.empty(3, 2 * T, dtype=torch.int32, device=META)[:, ::2],   # inner stride 2
    torch.empty(3, T, 1, dtype=torch.int32, device=META),
])
def test_bad_positions_are_refused(pos):
    with pytest.raises(ValueError, match="pos"):
        check_decode_layers([_layer()], pos)


def test_positions_on_another_device_are_refused():
    with pytest.raises(ValueError, match="device"):
        check_decode_layers([_layer()], torch.empty(3, T, dtype=torch.int32))


@pytest.mark.parametrize("n", [0, 3, 4])
def test_check_positions_counts_tokens(n):
    with pytest.raises(ValueError, match="fewer"):
        check_positions(_pos(n), 5)
    check_positions(_pos(5), 5)
    check_positions(_pos(5)[:, :5], 5)


def test_sliced_positions_of_a_longer_buffer():
    big = torch.empty(3, 100, dtype=torch.int32, device=META)
    check_positions(big[:, :40], 40)
    with pytest.raises(ValueError, match="fewer"):
        check_positions(big[:, :30], 40)
