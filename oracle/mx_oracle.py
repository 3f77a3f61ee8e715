"""CPU oracle for the MXFP6 block-scaled GEMM path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The library under
``microscaled_precision_gemm_amd/`` never imports it and shares no code with it.

It is the plain, slow, obviously-correct definition of what the GPU path
computes, in float64 with numpy:

* MXFP6 is the microscaled format the Hedra post "Optimizing Krea 3 on AMD
  Instinct MI355X with AI researchers" adopts for the DiT MLPs (section
  "Quality set the precision limit"): 6-bit floating-point elements that share
  one scale per block.  The pages fix neither the element variant, the block
  size, the scale encoding nor the rounding; this module follows the OCP
  Microscaling (MX) v1.0 definition: blocks of 32 elements along K, one E8M0
  power-of-two scale per block, elements E2M3 or E3M2, scale exponent
  ``floor(log2(amax)) - emax_elem``, round-to-nearest-even with saturation.
* The GEMM is ``C = A @ W.T`` on the dequantized operands, exact products and
  an fp64 sum; ``S = |A| @ |W|.T`` is the scale used by the tolerance.
* The fused fc1 epilogue is GELU with the tanh approximation (Hendrycks and
  Gimpel, "Gaussian Error Linear Units", 2016) followed by the same MX
  quantization, with blocks of 32 consecutive output columns.  In the Hedra
  post (section "Fusion cut intermediate memory traffic") fc2 takes fc1's
  output already in MXFP6, with no bf16 copy written and re-quantized in
  between; this function defines that MXFP6 operand.
* The SwiGLU variant of that epilogue (the MLP activation the same section
  names for Krea 3): the gate and up projections are one GEMM over stacked
  weights, and each output is silu(gate) * up (Shazeer, "GLU Variants Improve
  Transformer", 2020; silu(x) = x * sigmoid(x)), MX-quantized the same way.
  The stacking order is the library's own: in each run of 128 stacked rows,
  the first 64 are gate rows of 64 consecutive features, the next 64 the up
  rows of the same features.
* The quantize-once producer of the projection and MLP inputs (same section:
  modulation and RMSNorm fused, activations quantized once): RMSNorm (Zhang
  and Sennrich, "Root Mean Square Layer Normalization", 2019, with the usual
  eps inside the root) with a per-feature gain, then the adaptive-norm
  modulation of diffusion transformers (Peebles and Xie, "Scalable Diffusion
  Models with Transformers", 2023): y = norm(x) * (1 + scale) + shift, with
  one (shift, scale) pair of vectors per conditioning (sample), then MX
  quantization of y along the row.  The fused RMSNorm kernel of "Creating
  Custom Kernels for the AMD MI300" (section "Fused RMS Norm Kernel") is the
  MI300X counterpart.

* The format variants on the same scaled matrix instruction: the section
  "Quality set the precision limit" weighs MXFP4 (which the chip runs at the
  MXFP6 rate, rejected there on quality) and FP8 against MXFP6.  Their OCP MX
  element types are E2M1 (4 bits, max 6), E4M3 (8 bits, bias 7, max 448, the
  all-ones exponent and mantissa pattern is NaN, no infinity) and E5M2
  (8 bits, bias 15, max 57344, the all-ones exponent field is infinity or
  NaN).  The same scale rule and rounding apply; special codes are never
  produced (finite magnitudes above the largest saturate to it).

Readings where the pages are silent:

* all-zero block -> the scale exponent clamps to -127 (byte 0x00), codes +-0;
* the sign bit of each code is the sign bit of the source value, so -0.0 and
  negative values that round to zero give code 0b100000;
* a block holding a NaN or an infinity gets scale byte 0xFF (NaN) and codes 0;
* packing: element i of a 32-element block occupies bits [b*i, b*i+b) of a
  little-endian field of 32*b bits, b the element width (24 bytes for the
  6-bit types, 16 for E2M1 with element 2i in the low nibble of byte i, 32
  for the 8-bit types); blocks follow each other along a row.
"""

from __future__ import annotations

import numpy as np

BLOCK = 32
SCALE_NAN = 0xFF

# Element formats: exponent bits, mantissa bits, exponent bias.
FORMATS = {
    "e2m3": (2, 3, 1),   # FP6
    "e3m2": (3, 2, 3),   # FP6
    "e2m1": (2, 1, 1),   # FP4
    "e4m3": (4, 3, 7),   # FP8: exponent and mantissa all ones is NaN; no infinity
    "e5m2": (5, 2, 15),  # FP8: exponent all ones is infinity (mantissa 0) or NaN
}


def _fmt(fmt: str) -> tuple[int, int, int]:
    try:
        return FORMATS[fmt]
    except KeyError:
        raise ValueError(f"unknown MX element format {fmt!r}") from None


def element_bits(fmt: str) -> int:
    """Width of one element code: sign + exponent + mantissa bits."""
    ebits, mbits, _ = _fmt(fmt)
    return 1 + ebits + mbits


def element_values(fmt: str) -> np.ndarray:
    """Value of each of the 2**b element codes, decoded from the bit fields.

    Code bits: sign (top bit), exponent field e (E bits), mantissa field m
    (M bits).  e == 0 is subnormal: 2**(1-bias) * m / 2**M; otherwise
    2**(e-bias) * (1 + m / 2**M).  The 6-bit and 4-bit types have no special
    codes.  E4M3 reserves e and m all ones for NaN; E5M2 reserves e all ones
    for infinity (m == 0) and NaN.
    """
    ebits, mbits, bias = _fmt(fmt)
    bits = 1 + ebits + mbits
    vals = np.empty(1 << bits, dtype=np.float64)
    emask, mmask = (1 << ebits) - 1, (1 << mbits) - 1
    for c in range(1 << bits):
        sign = -1.0 if (c >> (bits - 1)) & 1 else 1.0
        e = (c >> mbits) & emask
        m = c & mmask
        if fmt == "e4m3" and e == emask and m == mmask:
            mag = np.nan
        elif fmt == "e5m2" and e == emask:
            mag = np.inf if m == 0 else np.nan
        elif e == 0:
            mag = 2.0 ** (1 - bias) * (m / 2.0 ** mbits)
        else:
            mag = 2.0 ** (e - bias) * (1.0 + m / 2.0 ** mbits)
        vals[c] = sign * mag
    return vals


def magnitudes(fmt: str) -> np.ndarray:
    """The finite non-negative magnitudes, indexed by code (codes 0 .. top):
    32 for the 6-bit types, 8 for E2M1, 127 for E4M3, 124 for E5M2."""
    pos = element_values(fmt)[: 1 << (element_bits(fmt) - 1)]
    return pos[np.isfinite(pos)].copy()


def floor_log2(x: np.ndarray) -> np.ndarray:
    """Exact floor(log2(x)) for finite x > 0 (float64 input).

    ``np.frexp`` splits x = f * 2**e with f in [0.5, 1) exactly, so
    floor(log2(x)) = e - 1 with no floating-point log involved.
    """
    _, e = np.frexp(np.asarray(x, dtype=np.float64))
    return e.astype(np.int64) - 1


def emax_elem(fmt: str) -> int:
    """Exponent of the largest normal element: floor(log2(max magnitude))."""
    return int(floor_log2(np.array([magnitudes(fmt).max()]))[0])


def e8m0_value(u) -> np.ndarray:
    """E8M0 scale byte -> 2**(u - 127); byte 0xFF is NaN."""
    u = np.asarray(u, dtype=np.int64)
    out = np.ldexp(1.0, u - 127)
    return np.where(u == SCALE_NAN, np.nan, out)


def round_to_code(r: np.ndarray, fmt: str) -> np.ndarray:
    """Nearest element code for already-scaled values r (float64).

    The magnitude goes to the nearest of the format's finite magnitudes; an
    exact tie goes to the even code (mantissa LSB 0), which is
    round-half-to-even because the codes increase with the magnitude.  A
    magnitude above the largest one maps to the largest (saturation), so the
    special codes of the 8-bit types never appear.  The sign bit is copied
    from r, so -0.0 and negative underflow give the negative-zero code.
    """
    mags = magnitudes(fmt)
    top = len(mags) - 1
    r = np.asarray(r, dtype=np.float64)
    a = np.abs(r)
    hi = np.searchsorted(mags, a, side="left")  # first magnitude >= a
    hi = np.minimum(hi, top)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    # above the largest magnitude: nearest is the largest
    pick = np.where(a >= mags[top], top, pick)
    sign = np.signbit(r).astype(np.int64)
    return (pick + (sign << (element_bits(fmt) - 1))).astype(np.uint8)


def quantize(x: np.ndarray, fmt: str = "e2m3") -> tuple[np.ndarray, np.ndarray]:
    """MX-quantize rows of x along the last axis in blocks of 32.

    x: float64 array [rows, K] holding the source values exactly (bf16 or
    fp32 values), K a multiple of 32.
    Returns (codes uint8 [rows, K], scales uint8 [rows, K/32]).

    Per block: amax = max |v|; shared = floor(log2 amax) - emax_elem clamped
    to [-127, 127] (amax == 0 clamps to -127); scale byte = shared + 127;
    each element is v / 2**shared rounded by ``round_to_code``.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] % BLOCK != 0:
        raise ValueError("quantize expects [rows, K] with K a multiple of 32")
    rows, k = x.shape
    blk = x.reshape(rows, k // BLOCK, BLOCK)
    finite = np.all(np.isfinite(blk), axis=2)
    safe = np.where(np.isfinite(blk), blk, 0.0)
    amax = np.max(np.abs(safe), axis=2)
    emax = emax_elem(fmt)
    with np.errstate(divide="ignore"):
        fl = np.where(amax > 0, floor_log2(np.where(amax > 0, amax, 1.0)), -100000)
    shared = np.clip(fl - emax, -127, 127)
    scales = np.where(finite, shared + 127, SCALE_NAN).astype(np.uint8)
    r = np.ldexp(safe, -shared[:, :, None])  # exact: a power-of-two scaling in float64
    codes = round_to_code(r, fmt).reshape(rows, k)
    codes = np.where(np.repeat(finite, BLOCK, axis=1), codes, 0).astype(np.uint8)
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str = "e2m3") -> np.ndarray:
    """codes [rows, K], scales [rows, K/32] -> float64 values [rows, K]."""
    codes = np.asarray(codes)
    rows, k = codes.shape
    vals = element_values(fmt)[codes.astype(np.int64)]
    sc = e8m0_value(np.asarray(scales))
    return (vals.reshape(rows, k // BLOCK, BLOCK) * sc[:, :, None]).reshape(rows, k)


def pack(codes: np.ndarray, fmt: str = "e2m3") -> np.ndarray:
    """codes uint8 [rows, K] -> packed bytes uint8 [rows, K*b/8], b the
    element width of fmt.

    Element i of the row occupies bits [b*i, b*i+b) of the row's
    little-endian bit string.  6 bits: four codes c0..c3 make the 24-bit word
    c0 | c1<<6 | c2<<12 | c3<<18 stored as three bytes, low byte first (a
    32-element block is 24 bytes).  4 bits: byte i is c[2i] | c[2i+1]<<4.
    8 bits: one byte per code.
    """
    codes = np.asarray(codes, dtype=np.uint32)
    rows, k = codes.shape
    bits = element_bits(fmt)
    if k % 4:
        raise ValueError("K must be a multiple of 4")
    if np.any(codes >= (1 << bits)):
        raise ValueError(f"codes must be {bits}-bit")
    if bits == 8:
        return codes.astype(np.uint8)
    if bits == 4:
        q = codes.reshape(rows, k // 2, 2)
        return (q[..., 0] | (q[..., 1] << 4)).astype(np.uint8)
    q = codes.reshape(rows, k // 4, 4)
    w = q[..., 0] | (q[..., 1] << 6) | (q[..., 2] << 12) | (q[..., 3] << 18)
    out = np.stack([w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF], axis=-1)
    return out.reshape(rows, 3 * k // 4).astype(np.uint8)


def unpack(packed: np.ndarray, k: int, fmt: str = "e2m3") -> np.ndarray:
    """Inverse of ``pack``: bytes [rows, K*b/8] -> codes uint8 [rows, K]."""
    packed = np.asarray(packed, dtype=np.uint32)
    rows = packed.shape[0]
    bits = element_bits(fmt)
    if packed.shape[1] != bits * k // 8:
        raise ValueError("packed width does not match K")
    if bits == 8:
        return packed.astype(np.uint8)
    if bits == 4:
        q = np.stack([packed & 15, packed >> 4], axis=-1)
        return q.reshape(rows, k).astype(np.uint8)
    b = packed.reshape(rows, k // 4, 3)
    w = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
    q = np.stack([(w >> (6 * i)) & 63 for i in range(4)], axis=-1)
    return q.reshape(rows, k).astype(np.uint8)


def gemm_ref(a: np.ndarray, w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """C = A @ W.T and S = |A| @ |W|.T in float64.

    a: [M, K] dequantized activations, w: [N, K] dequantized weights (the
    PyTorch Linear layout).  Every product of two MX values is exact in
    float64; the sum's rounding error is at most about K * 2**-53 * S.
    """
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return a @ w.T, np.abs(a) @ np.abs(w).T


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GELU, tanh form: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x**3).

    Evaluated as x / (1 + exp(-2u)), the same function (0.5 (1 + tanh u) is the
    logistic function of 2u), because 1 + tanh(u) cancels for negative u and
    would lose most digits of the small negative outputs.
    """
    x = np.asarray(x, dtype=np.float64)
    u = np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-2.0 * u))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    bf16 has 8 significant bits and fp32's exponent range: the spacing at
    |x| in [2**e, 2**(e+1)) is 2**(e-7), and 2**-133 below 2**-126.
    Results above the largest finite bf16 become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    e = np.where(fin, floor_log2(np.where(fin, np.abs(x), 1.0)), 0)
    q = np.maximum(e, -126) - 7
    rounded = np.ldexp(np.rint(np.ldexp(x, -q)), q)  # np.rint rounds half to even
    out = np.where(fin, rounded, out)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    out = np.where(np.abs(out) > bf16_max, np.copysign(np.inf, out), out)
    return out


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (2**-133 at and below the normal range)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.where(x > 0, floor_log2(np.where(x > 0, x, 1.0)), -126)
    return np.ldexp(1.0, np.maximum(e, -126) - 7)


def ulp_fp32(x: np.ndarray) -> np.ndarray:
    """Spacing of fp32 numbers at |x|."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.where(x > 0, floor_log2(np.where(x > 0, x, 1.0)), -126)
    return np.ldexp(1.0, np.maximum(e, -126) - 23)


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU (swish with beta 1): x * sigmoid(x) = x / (1 + exp(-x))."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


SWIGLU_RUN = 64  # gate rows, then as many up rows, per 128 stacked rows


def swiglu_rows(h: int) -> tuple[np.ndarray, np.ndarray]:
    """Stacked-weight row indices of the gate and of the up projection of
    features 0 .. h-1 (h a multiple of 64): feature f's gate row is
    128 * (f // 64) + f % 64 and its up row 64 rows later."""
    if h % SWIGLU_RUN:
        raise ValueError("the SwiGLU hidden size must be a multiple of 64")
    f = np.arange(h)
    gate = 2 * SWIGLU_RUN * (f // SWIGLU_RUN) + f % SWIGLU_RUN
    return gate, gate + SWIGLU_RUN


def swiglu_ref(a_deq: np.ndarray, w_stacked_deq: np.ndarray):
    """SwiGLU projection on dequantized operands: C = A @ Ws.T over the 2h
    stacked rows, then out[:, f] = silu(C[:, gate f]) * C[:, up f].

    Returns (out, gate, up, s_gate, s_up) in float64, where s_* are the
    |A| @ |W|.T scales of the gate and up columns (for the tolerance)."""
    c, s = gemm_ref(a_deq, w_stacked_deq)
    gi, ui = swiglu_rows(c.shape[1] // 2)
    gate, up = c[:, gi], c[:, ui]
    return silu(gate) * up, gate, up, s[:, gi], s[:, ui]


def fc1_swiglu_mx_ref(a_deq: np.ndarray, w_stacked_deq: np.ndarray, out_fmt: str = "e2m3"):
    """Stacked gate/up projection with the fused SwiGLU epilogue,
    re-quantized along the h output features from the fp32 rounding of the
    float64 result (the precision the device quantizes in).  Returns
    (codes [M, h], scales [M, h/32], out64, gate, up, s_gate, s_up)."""
    out, gate, up, sg, su = swiglu_ref(a_deq, w_stacked_deq)
    codes, scales = quantize(out.astype(np.float32).astype(np.float64), out_fmt)
    return codes, scales, out, gate, up, sg, su


def rmsnorm_modulate(x: np.ndarray, gamma=None, shift=None, scale=None, rows_per_cond: int | None = None,
                     eps: float = 1e-6) -> np.ndarray:
    """y[r] = x[r] / sqrt(mean(x[r]**2) + eps) * gamma * (1 + scale[c]) + shift[c],
    c = r // rows_per_cond, in float64.  gamma [d] (None = ones); shift and
    scale [n_cond, d] (None = zeros)."""
    x = np.asarray(x, dtype=np.float64)
    rows, d = x.shape
    inv = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    y = x * inv
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)[None, :]
    if scale is not None or shift is not None:
        per = rows if rows_per_cond is None else rows_per_cond
        c = np.arange(rows) // per
        if scale is not None:
            y = y * (1.0 + np.asarray(scale, dtype=np.float64)[c])
        if shift is not None:
            y = y + np.asarray(shift, dtype=np.float64)[c]
    return y


def rmsnorm_quantize_ref(x: np.ndarray, gamma=None, shift=None, scale=None, rows_per_cond=None, eps: float = 1e-6,
                         fmt: str = "e2m3"):
    """The producer's output: MX quantization of fp32(rmsnorm_modulate(x)).
    Returns (codes, scales, y64)."""
    y = rmsnorm_modulate(x, gamma, shift, scale, rows_per_cond, eps)
    codes, scales = quantize(y.astype(np.float32).astype(np.float64), fmt)
    return codes, scales, y


# ---------------------------------------------------------------------------
# Whole-path references, one per GEMM flavour the library exposes.
# ---------------------------------------------------------------------------

def linear_ref(a_deq: np.ndarray, w_deq: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Plain MX GEMM (fp32 / bf16 output flavours): exact C and the scale S."""
    return gemm_ref(a_deq, w_deq)


def fc1_gelu_mx_ref(a_deq: np.ndarray, w_deq: np.ndarray, out_fmt: str = "e2m3"):
    """fc1 with the fused epilogue: GELU-tanh of C, re-quantized along N.

    The GELU is evaluated in float64 on the exact C; the value handed to the
    quantizer is that result rounded to fp32, the precision the device
    epilogue quantizes in, so that both sides take the rounding decision on an
    fp32 number.  Returns (codes [M, N], scales [M, N/32], C, S, g64) where
    g64 is the float64 GELU before the fp32 rounding.
    """
    c, s = gemm_ref(a_deq, w_deq)
    g64 = gelu_tanh(c)
    g32 = g64.astype(np.float32).astype(np.float64)
    codes, scales = quantize(g32, out_fmt)
    return codes, scales, c, s, g64


# ---------------------------------------------------------------------------
# Tolerance checks (the parity bar).
# ---------------------------------------------------------------------------

GEMM_RTOL = 1e-5


def check_fp32(gpu: np.ndarray, c: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Boolean mask of fp32 outputs within |gpu - C| <= 1e-5 * S."""
    gpu = np.asarray(gpu, dtype=np.float64)
    return np.abs(gpu - c) <= GEMM_RTOL * s


def check_bf16(gpu: np.ndarray, c: np.ndarray, s: np.ndarray) -> tuple[np.ndarray, int]:
    """bf16 outputs: within 1 bf16 ulp of C, or, where |C| is far below S
    (cancellation), within 1e-5 * S + half a bf16 ulp of C.

    Returns (pass mask, number of elements that needed the second clause).
    """
    gpu = np.asarray(gpu, dtype=np.float64)
    d = np.abs(gpu - c)
    u = ulp_bf16(c)
    first = d <= u
    second = d <= GEMM_RTOL * s + 0.5 * u
    ok = first | second
    return ok, int(np.count_nonzero(second & ~first))
