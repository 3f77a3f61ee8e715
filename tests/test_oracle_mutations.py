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
_ORIG_E8M0 = O.e8m0_value
_ORIG_UNPACK = O.unpack
_ORIG_QUANTIZE = O.quantize
_ORIG_GEMM = O.gemm_ref


def _e8m0_bias_128(u):
    """The scale byte decoded with bias 128 instead of 127."""
    return _ORIG_E8M0(np.asarray(u).astype(np.int64) - 1)


def _unpack_msb_first(packed, k, fmt="e2m3"):
    """6-bit codes read from the top of each 24-bit word down."""
    if O.element_bits(fmt) != 6:
        return _ORIG_UNPACK(packed, k, fmt)
    packed = np.asarray(packed, dtype=np.uint32)
    rows = packed.shape[0]
    b = packed.reshape(rows, k // 4, 3)
    w = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
    q = np.stack([(w >> (6 * (3 - i))) & 63 for i in range(4)], axis=-1)
    return q.reshape(rows, k).astype(np.uint8)


def _rms_mean_over_rows(x, gamma=None, shift=None, scale=None, rows_per_cond=None, eps=1e-6):
    """The mean of squares taken down the columns instead of along the row."""
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=0, keepdims=True) + eps)
    if gamma is not None:
        y = y * np.asarray(gamma)[None, :]
    rows = x.shape[0]
    c = np.arange(rows) // (rows if rows_per_cond is None else rows_per_cond)
    if scale is not None:
        y = y * (1.0 + np.asarray(scale)[c])
    if shift is not None:
        y = y + np.asarray(shift)[c]
    return y


def _quantize_no_saturation(x, fmt="e2m3"):
    """Magnitudes above the largest element wrap to the zero code instead of
    clamping to it."""
    codes, scales = _ORIG_QUANTIZE(x, fmt)
    x = np.asarray(x, dtype=np.float64)
    rows, k = x.shape
    sc = O.e8m0_value(scales)
    r = np.abs(x.reshape(rows, k // 32, 32)) / sc[:, :, None]
    over = (r > O.magnitudes(fmt).max()).reshape(rows, k)
    half = 1 << (O.element_bits(fmt) - 1)
    return np.where(over, codes & half, codes).astype(np.uint8), scales


def _gemm_k_reversed_w(a, w):
    """W's K axis read in reverse (a transposed-index slip)."""
    return _ORIG_GEMM(a, np.asarray(w)[:, ::-1])


def _check_fp32_loose(gpu, c, s):
    return np.abs(np.asarray(gpu, dtype=np.float64) - c) <= 1e-4 * s


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
    ("e8m0_value", _e8m0_bias_128, [lambda: pins.test_exhaustive_round_trip("e2m3")]),
    ("unpack", _unpack_msb_first, [pins.test_pack_round_trip_random]),
    ("rmsnorm_modulate", _rms_mean_over_rows, [pins.test_rmsnorm_matches_torch]),
    ("quantize", _quantize_no_saturation, [pins.test_block_cases]),
    ("gemm_ref", _gemm_k_reversed_w,
     [lambda: pins.test_gemm_exact_integer_brute_force("e2m3", "e3m2", 4, 4, 32)]),
    ("check_fp32", _check_fp32_loose, [pins.test_tolerance_checks]),
]


@pytest.mark.parametrize("name,mutant,tests", MUTANTS, ids=[f"{m[0]}-{i}" for i, m in enumerate(MUTANTS)])
def test_pin_catches_mutant(monkeypatch, name, mutant, tests):
    monkeypatch.setattr(O, name, mutant)
    for t in tests:
        with pytest.raises(AssertionError):
            t()
