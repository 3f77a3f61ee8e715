"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin
catches each one.  Every mutant must make at least one pin test fail."""

import numpy as np
import pytest

import tests.test_oracle as pins
from oracle import mx_oracle as O


def _ties_away(r, fmt):
    mags = O.magnitudes(fmt)
    a = np.abs(np.asarray(r, dtype=np.float64))
    hi = np.minimum(np.searchsorted(mags, a, side="left"), 31)
    lo = np.maximum(hi - 1, 0)
    pick = np.where(a - mags[lo] < mags[hi] - a, lo, hi)
    pick = np.where(a >= mags[31], 31, pick)
    return (pick + 32 * np.signbit(r)).astype(np.uint8)


def _emax_plus_one(fmt):
    return {"e2m3": 3, "e3m2": 5}[fmt]


def _pack_big_endian(codes):
    codes = np.asarray(codes, dtype=np.uint32)
    rows, k = codes.shape
    q = codes.reshape(rows, k // 4, 4)
    w = (q[..., 0] << 18) | (q[..., 1] << 12) | (q[..., 2] << 6) | q[..., 3]
    out = np.stack([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], axis=-1)
    return out.reshape(rows, 3 * k // 4).astype(np.uint8)


def _gemm_no_transpose_abs(a, w):
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return a @ w.T, np.abs(a @ w.T)


def _gemm_swapped_scale(a, w):
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return np.abs(a) @ np.abs(w).T, a @ w.T


def _gelu_wrong_constant(x):
    x = np.asarray(x, dtype=np.float64)
    u = np.sqrt(2.0 / np.pi) * (x + 0.0447 * x ** 3)
    return x / (1.0 + np.exp(-2.0 * u))


def _silu_doubled(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-2.0 * x))


def _swiglu_rows_swapped(h):
    f = np.arange(h)
    gate = 128 * (f // 64) + f % 64
    return gate + 64, gate


def _swiglu_rows_contiguous(h):
    f = np.arange(h)
    return f, f + h


def _rms_eps_outside(x, gamma=None, shift=None, scale=None, rows_per_cond=None, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    y = x / (np.sqrt(np.mean(x * x, axis=1, keepdims=True)) + eps)
    return y * (1.0 if gamma is None else np.asarray(gamma)[None, :])


def _rms_scale_not_plus_one(x, gamma=None, shift=None, scale=None, rows_per_cond=None, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    if gamma is not None:
        y = y * np.asarray(gamma)[None, :]
    rows = x.shape[0]
    c = np.arange(rows) // (rows if rows_per_cond is None else rows_per_cond)
    if scale is not None:
        y = y * np.asarray(scale)[c]
    if shift is not None:
        y = y + np.asarray(shift)[c]
    return y


def _bias_off(fmt):
    e, m, b = {"e2m3": (2, 3, 1), "e3m2": (3, 2, 3)}[fmt]
    return (e, m, b + 1)


MUTANTS = [
    ("round_to_code", _ties_away, [pins.test_element_rounding_cases]),
    ("emax_elem", _emax_plus_one, [pins.test_block_cases]),
    ("pack", _pack_big_endian, [pins.test_pack_cases]),
    ("gemm_ref", _gemm_no_transpose_abs,
     [lambda: pins.test_gemm_exact_integer_brute_force("e2m3", "e2m3", 4, 4, 32)]),
    ("gemm_ref", _gemm_swapped_scale, [pins.test_gemm_one_hot_selects_columns]),
    ("gelu_tanh", _gelu_wrong_constant, [pins.test_gelu_matches_torch_tanh_gelu]),
    ("_fmt", _bias_off, [pins.test_magnitudes_match_literal_table]),
    ("silu", _silu_doubled, [pins.test_silu_matches_torch]),
    ("swiglu_rows", _swiglu_rows_swapped, [pins.test_swiglu_stacking_and_product]),
    ("swiglu_rows", _swiglu_rows_contiguous, [pins.test_swiglu_stacking_and_product]),
    ("rmsnorm_modulate", _rms_eps_outside, [pins.test_rmsnorm_matches_torch]),
    ("rmsnorm_modulate", _rms_scale_not_plus_one, [pins.test_modulation_per_condition]),
]


@pytest.mark.parametrize("name,mutant,tests", MUTANTS, ids=[f"{m[0]}-{i}" for i, m in enumerate(MUTANTS)])
def test_pin_catches_mutant(monkeypatch, name, mutant, tests):
    monkeypatch.setattr(O, name, mutant)
    for t in tests:
        with pytest.raises(AssertionError):
            t()
