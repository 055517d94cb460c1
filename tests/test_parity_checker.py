"""The parity checker itself (CPU): results the bars must reject are rejected.

A NaN compares false with every bound, so a checker that only asks
`worst > tol` lets a NaN output through; these cases plant such outputs and
expect an AssertionError, and check that matching results still pass.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from parity import check


def _ref(shape=(4, 16), seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("pairs", [False, True])
def test_matching_result_passes(dtype, pairs):
    r = _ref()
    y = torch.from_numpy(r).to(dtype)
    check("checker/ok", y, r, pairs=pairs)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("pairs", [False, True])
@pytest.mark.parametrize("bad", [float("nan"), float("inf"), float("-inf")])
def test_planted_nonfinite_output_fails(dtype, pairs, bad):
    r = _ref()
    y = torch.from_numpy(r).to(dtype)
    y[2, 5] = bad
    with pytest.raises(AssertionError):
        check("checker/planted", y, r, pairs=pairs)


def test_planted_nan_fails_under_a_scale():
    r = _ref()
    y = torch.from_numpy(r).float()
    y[0, 0] = float("nan")
    with pytest.raises(AssertionError):
        check("checker/scaled", y, r, scale=np.abs(r) + 1.0)


def test_nan_where_oracle_is_finite_fails_and_matching_nan_passes():
    r = _ref()
    r[1, 1] = np.nan
    y = torch.from_numpy(r).float()
    check("checker/nan-both", y, r)             # NaN expected and produced
    y2 = y.clone()
    y2[1, 1] = 0.0
    with pytest.raises(AssertionError):
        check("checker/nan-missing", y2, r)     # NaN expected, finite produced


def test_wrong_sign_infinity_fails():
    r = _ref()
    r[3, 3] = np.inf
    y = torch.from_numpy(r).float()
    check("checker/inf-both", y, r)
    y[3, 3] = -float("inf")
    with pytest.raises(AssertionError):
        check("checker/inf-sign", y, r)


def test_one_ulp_off_passes_and_a_large_error_fails():
    r = _ref()
    y = torch.from_numpy(r).float()
    check("checker/fp32-close", y, r)
    y[0, 3] *= 1.001
    with pytest.raises(AssertionError):
        check("checker/fp32-far", y, r)
