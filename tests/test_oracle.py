"""Pins for the CPU oracle: each check ties it to something other than itself.

* literal tables and hand-derived cases (tests/golden/), from the OCP MX v1.0
  element and scale definitions that the MXFP6 format on the pages follows;
* exhaustive enumeration (all 64 codes of both formats);
* brute force with exact rationals / Python integers on small inputs;
* library routines for the special cases (torch's GELU-tanh, torch's fp32 ->
  bf16 rounding);
* invariants of the scale rule (power-of-two shifts, range of amax/2**shared).
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import mx_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


# ---------------------------------------------------------------- element tables

def test_magnitudes_match_literal_table():
    for line in _golden_lines("mx_element_magnitudes.txt"):
        fmt, *vals = line.split()
        want = np.array([float(v) for v in vals])
        assert want.shape == (32,)
        np.testing.assert_array_equal(O.magnitudes(fmt), want)
        # negative half mirrors the positive half (code c+32 = -value(c))
        full = O.element_values(fmt)
        np.testing.assert_array_equal(full[32:], -want)
        assert math.copysign(1.0, full[32]) == -1.0  # code 32 is -0


@pytest.mark.parametrize("fmt,bits,emax,vmax,min_sub,min_norm,nfinite", [
    ("e2m3", 6, 2, 7.5, 0.125, 1.0, 32),
    ("e3m2", 6, 4, 28.0, 0.0625, 0.25, 32),
    ("e2m1", 4, 2, 6.0, 0.5, 1.0, 8),
    ("e4m3", 8, 8, 448.0, 2.0 ** -9, 2.0 ** -6, 127),
    ("e5m2", 8, 15, 57344.0, 2.0 ** -16, 2.0 ** -14, 124),
])
def test_format_constants(fmt, bits, emax, vmax, min_sub, min_norm, nfinite):
    mags = O.magnitudes(fmt)
    assert O.element_bits(fmt) == bits
    assert len(mags) == nfinite
    assert O.emax_elem(fmt) == emax
    assert mags.max() == vmax
    assert mags[1] == min_sub
    assert np.all(np.diff(mags) > 0), "codes must increase strictly with the magnitude"
    # smallest normal: exponent field 1, mantissa 0
    mbits = {"e2m3": 3, "e3m2": 2, "e2m1": 1, "e4m3": 3, "e5m2": 2}[fmt]
    assert mags[1 << mbits] == min_norm
    assert np.all(np.isfinite(O.element_values(fmt))) == (bits < 8)


def test_fp4_fp8_element_values_match_literal_table():
    for line in _golden_lines("fp4_fp8_element_values.txt"):
        fmt, code, val = line.split()
        got = O.element_values(fmt)[int(code)]
        want = float(val)
        if math.isnan(want):
            assert math.isnan(got), (fmt, code, got)
        else:
            assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), (fmt, code, got, want)


@pytest.mark.parametrize("fmt,dtype", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_decode_matches_torch(fmt, dtype):
    """All 256 FP8 codes decode as torch's float8 types decode them."""
    ref = torch.arange(256, dtype=torch.uint8).view(dtype).to(torch.float64).numpy()
    got = O.element_values(fmt)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(got[fin], ref[fin])
    np.testing.assert_array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


@pytest.mark.parametrize("fmt,dtype", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_rounding_matches_torch_cast(fmt, dtype):
    """Within the finite range, element rounding equals torch's fp32 -> float8
    cast (round to nearest even), ties and subnormals included."""
    rng = np.random.default_rng(31)
    vmax = O.magnitudes(fmt).max()
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-20, 17, 200000))).astype(np.float32)
    mids = (O.magnitudes(fmt)[:-1] + O.magnitudes(fmt)[1:]) / 2  # every exact tie
    x = np.concatenate([x, mids.astype(np.float32), -mids.astype(np.float32), np.float32([0.0, -0.0])])
    x = x[np.abs(x) <= vmax]
    ref = torch.from_numpy(x).to(dtype).view(torch.uint8).numpy()
    got = O.round_to_code(x.astype(np.float64), fmt)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (fmt, x[bad[:5]], got[bad[:5]], ref[bad[:5]])


ALL_FMTS = ["e2m3", "e3m2", "e2m1", "e4m3", "e5m2"]


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_exhaustive_round_trip(fmt):
    """Every finite code decodes and re-encodes to itself, in a block whose
    scale is fixed to 2**0 by a max-magnitude element (so the block scale byte
    is 127)."""
    vals = O.element_values(fmt)
    vmax = O.magnitudes(fmt).max()
    for c in np.flatnonzero(np.isfinite(vals)):
        blk = np.zeros((1, 32))
        blk[0, 0] = vmax
        blk[0, 5] = vals[c]
        codes, scales = O.quantize(blk, fmt)
        assert scales[0, 0] == 127
        assert codes[0, 5] == c, (fmt, c, codes[0, 5])
        back = O.dequantize(codes, scales, fmt)
        assert back[0, 5] == vals[c]
        assert math.copysign(1.0, back[0, 5]) == math.copysign(1.0, vals[c])


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("shift", [-120, -20, -1, 3, 60, 100])
def test_round_trip_under_any_scale(fmt, shift):
    """Scaling a block by 2**k changes only the scale byte (by k), never the codes."""
    vals = O.element_values(fmt)
    mags = O.magnitudes(fmt)
    vmax = mags.max()
    half = 1 << (O.element_bits(fmt) - 1)
    pick = np.linspace(1, len(mags) - 1, 31).round().astype(int)  # 31 finite codes spread over the range
    base = np.zeros((2, 32))
    base[:, 0] = vmax
    base[0, 1:] = vals[pick]
    base[1, 1:] = vals[half + pick]
    c0, s0 = O.quantize(base, fmt)
    scaled = np.ldexp(base, shift)  # scale bytes 7 .. 227: inside the E8M0 range, no clamp
    c1, s1 = O.quantize(scaled, fmt)
    np.testing.assert_array_equal(c0, c1)
    np.testing.assert_array_equal(s1.astype(int), s0.astype(int) + shift)


# ---------------------------------------------------------------- rounding

def test_element_rounding_cases():
    for line in _golden_lines("element_rounding_cases.txt"):
        fmt, r, want = line.split()
        got = O.round_to_code(np.array([float(r)]), fmt)[0]
        assert int(got) == int(want), (fmt, r, int(got), want)


def test_block_cases():
    for line in _golden_lines("block_cases.txt"):
        head, vals, codes = (p.strip() for p in line.split("|"))
        fmt, scale = head.split()
        v = [float(x) for x in vals.split()]
        c = [int(x) for x in codes.split()]
        blk = np.zeros((1, 32))
        blk[0, : len(v)] = v
        got_c, got_s = O.quantize(blk, fmt)
        assert int(got_s[0, 0]) == int(scale), (line, int(got_s[0, 0]))
        assert got_c[0, : len(c)].tolist() == c, (line, got_c[0, : len(c)].tolist())
        assert not np.any(got_c[0, len(c):] % (1 << (O.element_bits(fmt) - 1))), line  # zero padding stays +-0


def _brute_code(r: Fraction, fmt: str, negative: bool) -> int:
    """Exhaustive search over all finite magnitudes with exact rationals."""
    mags = [Fraction(x) for x in O.magnitudes(fmt)]
    a = abs(r)
    best = None
    for c, m in enumerate(mags):
        d = abs(a - m)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    return best[1] + ((1 << (O.element_bits(fmt) - 1)) if negative else 0)


def _brute_shared(amax: Fraction, emax: int) -> int:
    """The unique integer s with 2**(s+emax) <= amax < 2**(s+emax+1), by search."""
    if amax == 0:
        return -127
    s = -400
    while not (Fraction(2) ** (s + emax) <= amax < Fraction(2) ** (s + emax + 1)):
        s += 1
    return max(-127, min(127, s))


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_quantize_matches_exact_brute_force(fmt):
    rng = np.random.default_rng(7)
    emax = {"e2m3": 2, "e3m2": 4, "e2m1": 2, "e4m3": 8, "e5m2": 15}[fmt]
    # bf16-valued inputs over a wide range of magnitudes, incl. ties and zeros
    x = rng.standard_normal((24, 32)).astype(np.float32)
    x *= np.exp2(rng.integers(-40, 40, size=(24, 1))).astype(np.float32)
    x[3, :] = 0.0
    x[4, ::3] = -0.0
    x[5, :] = np.float32(2.0 ** -133) * rng.integers(-3, 4, size=32)  # bf16 subnormals
    x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    codes, scales = O.quantize(x, fmt)
    for i in range(x.shape[0]):
        fr = [Fraction(float(v)) for v in x[i]]
        s = _brute_shared(max(abs(v) for v in fr), emax)
        assert int(scales[i, 0]) == s + 127
        for j in range(32):
            want = _brute_code(fr[j] / Fraction(2) ** s, fmt, math.copysign(1.0, x[i, j]) < 0)
            assert int(codes[i, j]) == want, (fmt, i, j, x[i, j])


def test_scale_invariant_on_random_blocks():
    rng = np.random.default_rng(11)
    for fmt in ALL_FMTS:
        emax = O.emax_elem(fmt)
        x = rng.standard_t(3, size=(200, 64)) * np.exp2(rng.integers(-60, 60, size=(200, 1)))
        x = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
        _, scales = O.quantize(x, fmt)
        amax = np.abs(x).reshape(200, 2, 32).max(axis=2)
        shared = scales.astype(np.int64) - 127
        ratio = amax / np.ldexp(1.0, shared)
        assert np.all(ratio >= 2.0 ** emax) and np.all(ratio < 2.0 ** (emax + 1))


def test_nonfinite_block_gets_nan_scale():
    x = np.zeros((1, 64))
    x[0, 3] = np.inf
    x[0, 40] = 1.0
    codes, scales = O.quantize(x, "e2m3")
    assert scales[0, 0] == 0xFF and not codes[0, :32].any()
    assert scales[0, 1] == 125 and codes[0, 40] == 24
    assert np.isnan(O.e8m0_value(0xFF))


# ---------------------------------------------------------------- packing

def test_pack_cases():
    for line in _golden_lines("pack_cases.txt"):
        codes, hexbytes = (p.strip() for p in line.split("|"))
        c = np.array([[int(x) for x in codes.split()]], dtype=np.uint8)
        want = np.array([[int(h, 16) for h in hexbytes.split()]], dtype=np.uint8)
        np.testing.assert_array_equal(O.pack(c), want)
        np.testing.assert_array_equal(O.unpack(want, 32), c)


def test_pack_cases_fp4_fp8():
    for line in _golden_lines("pack_cases_fp4_fp8.txt"):
        fmt, codes, hexbytes = (p.strip() for p in line.split("|"))
        c = np.array([[int(x) for x in codes.split()]], dtype=np.uint8)
        want = np.array([[int(h, 16) for h in hexbytes.split()]], dtype=np.uint8)
        assert c.shape == (1, 32) and want.shape == (1, O.element_bits(fmt) * 4)
        np.testing.assert_array_equal(O.pack(c, fmt), want)
        np.testing.assert_array_equal(O.unpack(want, 32, fmt), c)


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_pack_round_trip_random_fp4_fp8(fmt):
    rng = np.random.default_rng(4)
    bits = O.element_bits(fmt)
    c = rng.integers(0, 1 << bits, size=(5, 96), dtype=np.uint8)
    p = O.pack(c, fmt)
    assert p.shape == (5, 96 * bits // 8)
    np.testing.assert_array_equal(O.unpack(p, 96, fmt), c)


def test_pack_round_trip_random():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 64, size=(7, 96), dtype=np.uint8)
    p = O.pack(c)
    assert p.shape == (7, 72)
    np.testing.assert_array_equal(O.unpack(p, 96), c)


# ---------------------------------------------------------------- GEMM

# (exponent bits, mantissa bits, bias) written from the OCP MX element
# definitions, independently of the oracle's table
_BITFIELDS = {"e2m3": (2, 3, 1), "e3m2": (3, 2, 3), "e2m1": (2, 1, 1), "e4m3": (4, 3, 7), "e5m2": (5, 2, 15)}


def _int_decode(code: int, fmt: str) -> int:
    """Integer n with value = n * 2**-F, F = bias + M - 1 (E2M3: 3, E3M2: 4,
    E2M1: 1, E4M3: 9, E5M2: 16), from the bits."""
    eb, mb, _ = _BITFIELDS[fmt]
    s = -1 if (code >> (eb + mb)) & 1 else 1
    e, m = (code >> mb) & ((1 << eb) - 1), code & ((1 << mb) - 1)
    n = m if e == 0 else ((1 << mb) + m) << (e - 1)
    return s * n


def _finite_codes(fmt: str) -> np.ndarray:
    """Codes that are neither Inf nor NaN, from the bit fields."""
    eb, mb, _ = _BITFIELDS[fmt]
    c = np.arange(1 << (1 + eb + mb))
    e, m = (c >> mb) & ((1 << eb) - 1), c & ((1 << mb) - 1)
    if fmt == "e4m3":
        return c[~((e == 15) & (m == 7))]
    if fmt == "e5m2":
        return c[e != 31]
    return c


@pytest.mark.parametrize("fa,fw", [("e2m3", "e2m3"), ("e2m3", "e3m2"), ("e3m2", "e3m2"), ("e2m1", "e2m1"),
                                   ("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e5m2", "e5m2"), ("e2m1", "e4m3")])
@pytest.mark.parametrize("m,n,k", [(4, 4, 32), (3, 5, 64), (2, 3, 96)])
def test_gemm_exact_integer_brute_force(fa, fw, m, n, k):
    rng = np.random.default_rng([m, n, k, len(fa + fw), ord(fa[1]), ord(fw[1])])
    ca = rng.choice(_finite_codes(fa), size=(m, k)).astype(np.uint8)
    cw = rng.choice(_finite_codes(fw), size=(n, k)).astype(np.uint8)
    sa = rng.integers(110, 145, size=(m, k // 32), dtype=np.uint8)
    sw = rng.integers(110, 145, size=(n, k // 32), dtype=np.uint8)
    frac = {f: b + mb - 1 for f, (_, mb, b) in _BITFIELDS.items()}
    c_ref, s_ref = O.gemm_ref(O.dequantize(ca, sa, fa), O.dequantize(cw, sw, fw))
    for i in range(m):
        for j in range(n):
            exact = Fraction(0)
            absum = Fraction(0)
            for b in range(k // 32):
                acc = 0
                aacc = 0
                for t in range(32 * b, 32 * b + 32):
                    p = _int_decode(int(ca[i, t]), fa) * _int_decode(int(cw[j, t]), fw)
                    acc += p
                    aacc += abs(p)
                sc = Fraction(2) ** (int(sa[i, b]) + int(sw[j, b]) - 254 - frac[fa] - frac[fw])
                exact += acc * sc
                absum += aacc * sc
            assert abs(Fraction(float(c_ref[i, j])) - exact) <= Fraction(1, 10 ** 12) * absum
            assert abs(Fraction(float(s_ref[i, j])) - absum) <= Fraction(1, 10 ** 12) * absum


def test_gemm_one_hot_selects_columns():
    """W rows that are one-hot pick single columns of A times both scales;
    guards against a transposed operand or a dropped scale."""
    rng = np.random.default_rng(5)
    k = 64
    ca = rng.integers(0, 64, size=(3, k), dtype=np.uint8)
    sa = rng.integers(120, 135, size=(3, 2), dtype=np.uint8)
    a = O.dequantize(ca, sa, "e2m3")
    cw = np.zeros((4, k), dtype=np.uint8)
    cols = [0, 17, 40, 63]
    for j, col in enumerate(cols):
        cw[j, col] = 8  # 1.0
    sw = np.full((4, 2), 129, dtype=np.uint8)  # x4
    c, s = O.gemm_ref(a, O.dequantize(cw, sw, "e2m3"))
    for j, col in enumerate(cols):
        np.testing.assert_array_equal(c[:, j], 4.0 * a[:, col])
        np.testing.assert_array_equal(s[:, j], 4.0 * np.abs(a[:, col]))


# ---------------------------------------------------------------- GELU

def test_gelu_matches_torch_tanh_gelu():
    x = np.concatenate([np.linspace(-12, 12, 4801), np.random.default_rng(2).standard_normal(5000) * 4])
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    # torch evaluates 1 + tanh(u), which cancels for negative u: allow its
    # absolute error there (about 1e-16 * |x|)
    err = np.abs(O.gelu_tanh(x) - ref)
    assert np.all(err <= 1e-13 * np.abs(ref) + 4e-16 * np.maximum(1.0, np.abs(x)))


def test_gelu_identities():
    x = np.linspace(-20, 20, 8001)
    g = O.gelu_tanh(x)
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(g - O.gelu_tanh(-x), x, atol=1e-12)  # odd part is x/2
    big = np.array([10.0, 30.0])
    np.testing.assert_array_equal(O.gelu_tanh(big), big)  # tanh saturates to 1
    # equivalent logistic form x * sigmoid(2u)
    u = np.sqrt(2 / np.pi) * (x + 0.044715 * x ** 3)
    np.testing.assert_allclose(g, x / (1 + np.exp(-2 * u)), rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- bf16 rounding / tolerance

def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-140, 120, 200000))).astype(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_ties_and_ulp():
    one = 1.0
    assert O.round_bf16(np.array([one + 2 ** -8]))[0] == 1.0  # tie, even
    assert O.round_bf16(np.array([one + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6  # tie, even
    assert O.round_bf16(np.array([one + 2 ** -8 + 2 ** -40]))[0] == 1.0 + 2 ** -7
    assert O.ulp_bf16(np.array([1.0]))[0] == 2 ** -7
    assert O.ulp_bf16(np.array([1.99]))[0] == 2 ** -7
    assert O.ulp_bf16(np.array([2.0 ** -130]))[0] == 2 ** -133
    assert O.ulp_fp32(np.array([1.0]))[0] == 2 ** -23


def test_tolerance_checks():
    c = np.array([1.0, 1.0, 1e-6])
    s = np.array([1.0, 1.0, 10.0])
    ok, n2 = O.check_bf16(np.array([1.0 + 2 ** -7, 1.0 + 2 ** -6, 5e-5]), c, s)
    assert ok.tolist() == [True, False, True] and n2 == 1
    assert O.check_fp32(np.array([1.0 + 1e-6, 1.0 + 2e-5, 0.0]), c, s).tolist() == [True, False, True]


def test_fc1_reference_is_quantized_gelu():
    rng = np.random.default_rng(4)
    a = O.dequantize(*O.quantize(rng.standard_normal((8, 64)), "e2m3"), "e2m3")
    w = O.dequantize(*O.quantize(rng.standard_normal((64, 64)) * 0.05, "e2m3"), "e2m3")
    codes, scales, c, s, g = O.fc1_gelu_mx_ref(a, w)
    assert codes.shape == (8, 64) and scales.shape == (8, 2)
    deq = O.dequantize(codes, scales, "e2m3")
    g32 = g.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(g, O.gelu_tanh(c))
    # each output lies within half an element spacing (at its block scale) of
    # fp32(GELU(C)); a value above 7.5 scale units saturates to 7.5
    unit = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    r = np.abs(g32) / unit
    spacing = np.ldexp(1.0, np.maximum(O.floor_log2(np.where(r > 0, r, 1.0)), 0) - 3)
    allowed = np.where(r > 7.5, r - 7.5, 0.5 * spacing) * unit
    assert np.all(np.abs(deq - g32) <= allowed * (1 + 1e-12))


# ---------------------------------------------------------------- SwiGLU

def test_silu_matches_torch():
    x = np.concatenate([np.linspace(-60, 60, 6001), np.random.default_rng(5).standard_normal(5000) * 6])
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(O.silu(x), ref, rtol=1e-14, atol=1e-300)


def test_silu_identities():
    x = np.linspace(-30, 30, 6001)
    assert O.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.silu(x) - O.silu(-x), x, atol=1e-12)  # x sigma(x) - (-x) sigma(-x) = x
    assert O.silu(np.array([800.0]))[0] == 800.0
    assert O.silu(np.array([-800.0]))[0] == 0.0  # -800 / (1 + e^800) underflows to -0
    # minimum of x sigma(x) is about -0.27846 near x = -1.27846
    assert abs(O.silu(np.linspace(-3, 0, 300001)).min() + 0.2784645) < 1e-6


def test_swiglu_stacking_and_product():
    """A stacked weight built by interleaving blocks of 64 gate rows and 64 up
    rows gives silu(A Wg^T) * (A Wu^T), computed here with torch."""
    rng = np.random.default_rng(11)
    m, k, h = 5, 64, 192
    a = O.dequantize(*O.quantize(rng.standard_normal((m, k)), "e2m3"), "e2m3")
    wg = O.dequantize(*O.quantize(rng.standard_normal((h, k)) * 0.2, "e2m3"), "e2m3")
    wu = O.dequantize(*O.quantize(rng.standard_normal((h, k)) * 0.2, "e2m3"), "e2m3")
    ws = np.stack([wg.reshape(h // 64, 64, k), wu.reshape(h // 64, 64, k)], axis=1).reshape(2 * h, k)
    out, gate, up, sg, su = O.swiglu_ref(a, ws)
    ta, tg, tu = (torch.from_numpy(v) for v in (a, wg, wu))
    want = (torch.nn.functional.silu(ta @ tg.T) * (ta @ tu.T)).numpy()
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(sg, np.abs(a) @ np.abs(wg).T, rtol=1e-14)
    np.testing.assert_allclose(su, np.abs(a) @ np.abs(wu).T, rtol=1e-14)


def test_fc1_swiglu_reference_is_quantized_product():
    rng = np.random.default_rng(12)
    a = O.dequantize(*O.quantize(rng.standard_normal((8, 64)), "e2m3"), "e2m3")
    ws = O.dequantize(*O.quantize(rng.standard_normal((128, 64)) * 0.1, "e2m3"), "e2m3")
    codes, scales, out, gate, up, sg, su = O.fc1_swiglu_mx_ref(a, ws)
    assert codes.shape == (8, 64) and scales.shape == (8, 2)
    o32 = out.astype(np.float32).astype(np.float64)
    deq = O.dequantize(codes, scales, "e2m3")
    unit = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    r = np.abs(o32) / unit
    spacing = np.ldexp(1.0, np.maximum(O.floor_log2(np.where(r > 0, r, 1.0)), 0) - 3)
    allowed = np.where(r > 7.5, r - 7.5, 0.5 * spacing) * unit
    assert np.all(np.abs(deq - o32) <= allowed * (1 + 1e-12))


# ---------------------------------------------------------------- RMSNorm + modulation producer

def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((7, 96)) * np.exp2(rng.integers(-6, 6, (7, 1)))
    g = rng.standard_normal(96)
    for eps in (1e-6, 1e-2):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps).numpy()
        np.testing.assert_allclose(O.rmsnorm_modulate(x, g, eps=eps), ref, rtol=1e-13, atol=1e-15)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(22)
    x = rng.standard_normal((5, 128))
    y = O.rmsnorm_modulate(x, eps=0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)  # unit root mean square
    np.testing.assert_allclose(O.rmsnorm_modulate(3.5 * x, eps=0.0), y, rtol=1e-13)  # scale invariant
    np.testing.assert_allclose(O.rmsnorm_modulate(-x, eps=0.0), -y, rtol=1e-13)


def test_modulation_per_condition():
    """y = norm(x) * (1 + scale[c]) + shift[c] with c = row // rows_per_cond,
    checked row by row against torch's rms_norm."""
    rng = np.random.default_rng(23)
    rows, d, per = 6, 64, 2
    x = rng.standard_normal((rows, d))
    g = rng.standard_normal(d)
    sh = rng.standard_normal((rows // per, d))
    sc = rng.standard_normal((rows // per, d))
    y = O.rmsnorm_modulate(x, g, sh, sc, per, eps=1e-5)
    for r in range(rows):
        n = torch.nn.functional.rms_norm(torch.from_numpy(x[r:r + 1]), (d,), torch.from_numpy(g), 1e-5).numpy()[0]
        np.testing.assert_allclose(y[r], n * (1 + sc[r // per]) + sh[r // per], rtol=1e-13, atol=1e-14)
    # zero modulation is the plain norm
    np.testing.assert_allclose(O.rmsnorm_modulate(x, g, np.zeros((3, d)), np.zeros((3, d)), per),
                               O.rmsnorm_modulate(x, g), rtol=0, atol=0)


def test_rmsnorm_quantize_reference():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((4, 64))
    codes, scales, y = O.rmsnorm_quantize_ref(x)
    ref_codes, ref_scales = O.quantize(y.astype(np.float32).astype(np.float64), "e2m3")
    assert np.array_equal(codes, ref_codes) and np.array_equal(scales, ref_scales)
