"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin
catches each one.  Every mutant must make at least one pin test fail."""

import numpy as np
import pytest

import tests.test_oracle as pins
from oracle import mx_oracle as O


_ORIG_EMAX = O.emax_elem
_ORIG_FMT = O._fmt
_ORIG_VALUES = O.element_values


def _ties_away(r, fmt):
    mags = O.magnitudes(fmt)
    top = len(mags) - 1
    a = np.abs(np.asarray(r, dtype=np.float64))
    hi = np.minimum(np.searchsorted(mags, a, side="left"), top)
    lo = np.maximum(hi - 1, 0)
    pick = np.where(a - mags[lo] < mags[hi] - a, lo, hi)
    pick = np.where(a >= mags[top], top, pick)
    return (pick + (np.signbit(r).astype(np.int64) << (O.element_bits(fmt) - 1))).astype(np.uint8)


def _emax_plus_one(fmt):
    return _ORIG_EMAX(fmt) + 1


def _e4m3_nan_as_number(fmt):
    """Decode E4M3's NaN code as if it were the finite 480."""
    v = _ORIG_VALUES(fmt)
    if fmt == "e4m3":
        v = v.copy()
        v[127], v[255] = 480.0, -480.0
    return v


def _fp4_nibbles_swapped(codes, fmt="e2m3"):
    codes = np.asarray(codes, dtype=np.uint32)
    if O.element_bits(fmt) != 4:
        return _ORIG_PACK(codes, fmt)
    q = codes.reshape(codes.shape[0], -1, 2)
    return ((q[..., 0] << 4) | q[..., 1]).astype(np.uint8)


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
    e, m, b = _ORIG_FMT(fmt)
    return (e, m, b + 1)


_ORIG_PACK = O.pack


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
    ("element_values", _e4m3_nan_as_number,
     [lambda: pins.test_format_constants("e4m3", 8, 8, 448.0, 2.0 ** -9, 2.0 ** -6, 127),
      lambda: pins.test_fp8_decode_matches_torch("e4m3", pins.torch.float8_e4m3fn)]),
    ("pack", _fp4_nibbles_swapped, [pins.test_pack_cases_fp4_fp8]),
    ("emax_elem", _emax_plus_one, [lambda: pins.test_quantize_matches_exact_brute_force("e5m2")]),
]


@pytest.mark.parametrize("name,mutant,tests", MUTANTS, ids=[f"{m[0]}-{i}" for i, m in enumerate(MUTANTS)])
def test_pin_catches_mutant(monkeypatch, name, mutant, tests):
    monkeypatch.setattr(O, name, mutant)
    for t in tests:
        with pytest.raises(AssertionError):
            t()
