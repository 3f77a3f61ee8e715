"""Helpers for the GPU parity tests: oracle-side references and comparisons.

The oracle side only ever sees the seeded host inputs; GPU results are only
compared against it, never fed into it.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import mx_oracle as O


def say(msg: str) -> None:
    """Name the case before a GPU step (and flush), so a hang or fault names it."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def oracle_mx(x64: np.ndarray, fmt: str):
    """Oracle quantization of float64 source values: (codes, scales, dequantized)."""
    codes, scales = O.quantize(x64, fmt)
    return codes, scales, O.dequantize(codes, scales, fmt)


def tiled_chunk_offsets(bits: int = 6) -> np.ndarray:
    """offsets[j, b]: where byte b of row j's packed slice of a 128-element
    stage (16 * bits bytes: four blocks of 4 * bits bytes) sits inside its
    tiled chunk of 512 * bits bytes, as the library's header defines the
    layout.  Half h (blocks 2h and 2h+1) owns bytes [256 bits h, 256 bits
    (h+1)).  6 bits: plane A (bytes 0..15 of block 2h, 16 per row), plane L
    (its bytes 16..23, 8 per row), plane H (bytes 0..7 of block 2h+1, 8 per
    row), plane B (its bytes 8..23, 16 per row).  4 bits: planes of 16 bytes
    per row, block 2h then block 2h+1.  8 bits: half h holds bytes 16h..16h+15
    of blocks 0, 2, 1, 3 in four planes of 16 bytes per row."""
    eb = 4 * bits
    off = np.empty((32, 4 * eb), dtype=np.int64)
    for j in range(32):
        for b in range(4 * eb):
            q, t = divmod(b, eb)
            base = (q >> 1) * 256 * bits
            if bits == 6:
                if q % 2 == 0:
                    off[j, b] = base + (j * 16 + t if t < 16 else 512 + j * 8 + (t - 16))
                else:
                    off[j, b] = base + (768 + j * 8 + t if t < 8 else 1024 + j * 16 + (t - 8))
            elif bits == 4:
                off[j, b] = (q >> 1) * 1024 + (q % 2) * 512 + j * 16 + t
            else:
                hh = t // 16  # bytes 0..15 in half 0, 16..31 in half 1
                off[j, b] = hh * 2048 + (2 * (q % 2) + (q >> 1)) * 512 + j * 16 + t % 16
    return off


_CHUNK_OFFSETS = {b: tiled_chunk_offsets(b) for b in (4, 6, 8)}


def tiled_to_rows(codes_t: np.ndarray, scales_t: np.ndarray, rows: int, k: int, bits: int = 6):
    """Rearrange the tiled MX layout (128-element stages x 32-row groups, as the
    library's header defines it) into row-major packed codes [rows, bits*k/8]
    and scales [rows, k/32].  Also returns the padding (codes and scale bytes
    of rows >= rows or blocks >= k/32), which must be 0 and 127."""
    stages, groups = -(-k // 128), -(-rows // 32)
    row_bytes = 16 * bits  # packed bytes of one row of a stage
    c = np.asarray(codes_t).reshape(stages, groups, 512 * bits)[:, :, _CHUNK_OFFSETS[bits]]
    c = c.transpose(1, 2, 0, 3).reshape(groups * 32, stages * row_bytes)
    s = np.asarray(scales_t).reshape(stages, groups, 32, 4)       # [stage, group, row, block]
    s = s.transpose(1, 2, 0, 3).reshape(groups * 32, stages * 4)
    kb = bits * k // 8
    pad_c = np.concatenate([c[rows:].ravel(), c[:rows, kb:].ravel()])
    pad_s = np.concatenate([s[rows:].ravel(), s[:rows, k // 32:].ravel()])
    return c[:rows, :kb], s[:rows, :k // 32], pad_c, pad_s


def mx_rows_gather(gpu_mx, rows) -> tuple[np.ndarray, np.ndarray]:
    """Row-major packed codes [len(rows), bits*k/8] and scales [len(rows), k/32]
    of the given rows of an MXTensor in the tiled layout, gathered where the
    tensor lives: only those rows' bytes are copied to the host (for matrices
    of many GiB).  Same result as tiled_to_rows on the whole tensor, then
    [rows]."""
    bits = O.element_bits(gpu_mx.fmt)
    stages, groups = -(-gpu_mx.k // 128), -(-gpu_mx.rows // 32)
    rows = np.asarray(rows, dtype=np.int64)
    grp, j = rows // 32, rows % 32
    chunk = np.arange(stages, dtype=np.int64)[None, :] * groups + grp[:, None]          # [R, stages]
    cidx = chunk[:, :, None] * (512 * bits) + _CHUNK_OFFSETS[bits][j][:, None, :]       # [R, stages, 16 bits]
    sidx = (chunk[:, :, None] * 32 + j[:, None, None]) * 4 + np.arange(4)               # [R, stages, 4]
    dev = gpu_mx.codes.device
    c = gpu_mx.codes.reshape(-1)[torch.from_numpy(cidx.reshape(-1)).to(dev)]
    sc = gpu_mx.scales.reshape(-1)[torch.from_numpy(sidx.reshape(-1)).to(dev)]
    c = to_np(c).reshape(len(rows), stages * 16 * bits)
    sc = to_np(sc).reshape(len(rows), stages * 4)
    return c[:, :bits * gpu_mx.k // 8], sc[:, :gpu_mx.k // 32]


def mx_rows_view(gpu_mx):
    """Row-major (codes, scales) of a GPU MXTensor, checking tiled padding."""
    gc, gs = to_np(gpu_mx.codes), to_np(gpu_mx.scales)
    if gpu_mx.layout == "tiled":
        gc, gs, pad_c, pad_s = tiled_to_rows(gc, gs, gpu_mx.rows, gpu_mx.k, O.element_bits(gpu_mx.fmt))
        assert not pad_c.any(), "tiled padding codes must be 0"
        assert np.all(pad_s == 127), "tiled padding scales must be 127"
    return gc, gs


def assert_mx_equal(gpu_mx, codes_o: np.ndarray, scales_o: np.ndarray, what: str, rows=None) -> None:
    """GPU packed codes + scales must equal the oracle's bit for bit."""
    gc, gs = mx_rows_view(gpu_mx)
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    k = codes_o.shape[1]
    packed_o = O.pack(codes_o, gpu_mx.fmt)
    bad_s = np.argwhere(gs != scales_o)
    assert bad_s.size == 0, f"{what}: {len(bad_s)} scale bytes differ, first {bad_s[:5].tolist()}"
    if not np.array_equal(gc, packed_o):
        cg = O.unpack(gc, k, gpu_mx.fmt)
        bad = np.argwhere(cg != codes_o)
        raise AssertionError(f"{what}: {len(bad)} codes differ, first {bad[:5].tolist()} "
                             f"gpu {[int(cg[tuple(b)]) for b in bad[:5]]} oracle {[int(codes_o[tuple(b)]) for b in bad[:5]]}")


def assert_fp32_close(gpu: np.ndarray, c: np.ndarray, s: np.ndarray, what: str) -> None:
    ok = O.check_fp32(gpu, c, s)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} fp32 outputs outside 1e-5*S; first {i}: "
                             f"gpu {gpu[i]!r} oracle {c[i]!r} S {s[i]!r}")


def assert_bf16_close(gpu: np.ndarray, c: np.ndarray, s: np.ndarray, what: str) -> int:
    ok, n2 = O.check_bf16(gpu, c, s)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} bf16 outputs outside tolerance; first {i}: "
                             f"gpu {gpu[i]!r} oracle {c[i]!r} S {s[i]!r}")
    return n2


def bf16_tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


GELU_DERIV_MAX = 1.13  # max |d/dx GELU_tanh(x)| is about 1.129


def gelu_eval_slack(c: np.ndarray, g: np.ndarray) -> np.ndarray:
    """Bound on the fp32 device GELU's own error at exact input c: a few ulps of
    g plus the exp2 argument's rounding amplified by |argument| (relative error
    of 2^a is |a| ln2 times that of a)."""
    arg = 2.0 * np.sqrt(2.0 / np.pi) * np.log2(np.e) * np.abs(c) * (1.0 + 0.044715 * c * c)
    return (8.0 + 1.2 * arg) * O.ulp_fp32(g) + 1e-44


SILU_DERIV_MAX = 1.1  # max |d/dx silu(x)| is about 1.0998


def swiglu_bound(gate: np.ndarray, up: np.ndarray, s_gate: np.ndarray, s_up: np.ndarray,
                 out: np.ndarray) -> np.ndarray:
    """Distance the device's fp32 silu(gate) * up may lie from the exact value:
    the gate / up accumulation errors (<= 1e-5 S each) through the product's
    partial derivatives (|silu'| <= 1.1 times |up|, and |silu(gate)|), plus the
    fp32 evaluation of silu (its exp2 argument's rounding grows with |gate|)."""
    acc = O.GEMM_RTOL * (SILU_DERIV_MAX * np.abs(up) * s_gate + np.abs(O.silu(gate)) * s_up)
    return acc + (8.0 + 1.2 * np.abs(gate)) * O.ulp_fp32(out) + 1e-44


def rmsnorm_bound(x: np.ndarray, gamma, scale, rows_per_cond, eps: float, y: np.ndarray) -> np.ndarray:
    """Distance the device's fp32 RMSNorm + modulation may lie from the exact y:
    the sum of squares is accumulated per lane over d/64 terms and then over a
    64-lane tree (relative error <= (d/64 + 6) 2^-24), the root and the
    reciprocal add an ulp each, and the products x * inv * gamma * (1 + scale)
    three more roundings; the final fma rounds once (an ulp of y)."""
    x = np.asarray(x, dtype=np.float64)
    rows, d = x.shape
    inv = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    a = np.ones(d) if gamma is None else np.abs(np.asarray(gamma, dtype=np.float64))
    t = np.abs(x) * inv * a[None, :]
    if scale is not None:
        c = np.arange(rows) // rows_per_cond
        t = t * np.abs(1.0 + np.asarray(scale, dtype=np.float64)[c])
    rel = (d / 64 + 6 + 2 + 4) * 2.0 ** -24
    return t * rel + O.ulp_fp32(y) + 1e-44


def check_mx_epilogue(gpu_codes: np.ndarray, gpu_scales: np.ndarray, c: np.ndarray, s: np.ndarray, gelu: bool,
                      fmt: str = "e2m3") -> dict:
    """Compare a fused-epilogue MX output (GELU or identity, then MX along N)
    with the oracle.

    The oracle quantizes fp32(epilogue(C_exact)); the device quantizes its own
    fp32 result, which differs from that by the accumulation error (<= 1e-5 S,
    times |GELU'| <= 1.13) plus the GELU evaluation error.  Where the oracle's
    value is within that distance delta of a rounding midpoint, one element
    step either way is a correct result; where the block's amax is within delta
    of a power of two, the scale byte may differ by one.  Everything else must
    match exactly.  Returns counts of exact and tolerated differences.
    """
    g32, delta = mx_epilogue_target(c, s, gelu)
    return check_mx_values(gpu_codes, gpu_scales, g32, delta, fmt)


def mx_epilogue_target(c: np.ndarray, s: np.ndarray, gelu: bool) -> tuple[np.ndarray, np.ndarray]:
    """The oracle's fp32 epilogue value fp32(GELU(C)) (or fp32(C)) and the
    distance delta the device's fp32 value may lie from it."""
    g64 = O.gelu_tanh(c) if gelu else c
    g32 = g64.astype(np.float32).astype(np.float64)
    delta = O.GEMM_RTOL * s * (GELU_DERIV_MAX if gelu else 1.0) + (gelu_eval_slack(c, g32) if gelu else 0.0)
    return g32, delta


def check_mx_values(gpu_codes: np.ndarray, gpu_scales: np.ndarray, g32: np.ndarray, delta: np.ndarray,
                    fmt: str = "e2m3") -> dict:
    """The boundary-aware comparison of a fused MX output with the oracle's
    quantization of its fp32 values g32, given the distance delta by which the
    device's fp32 values may differ from them (see check_mx_epilogue)."""
    n = g32.shape[1]
    codes_o, scales_o = O.quantize(g32, fmt)
    codes_g = O.unpack(gpu_codes, n)
    deq_o = O.dequantize(codes_o, scales_o, fmt)
    deq_g = O.dequantize(codes_g, gpu_scales, fmt)
    delta = delta + O.ulp_fp32(g32)  # the oracle's own fp32 rounding of g
    rows, nb = scales_o.shape
    su_o = scales_o.astype(np.int64)
    su_g = gpu_scales.astype(np.int64)
    emax = O.emax_elem(fmt)
    mags = O.magnitudes(fmt)

    stats = {"elements": codes_o.size, "code_steps": 0, "scale_steps": 0, "exact": 0}
    # --- scales
    diff_s = su_g != su_o
    if diff_s.any():
        amax = np.abs(g32).reshape(rows, nb, 32).max(axis=2)
        dblk = delta.reshape(rows, nb, 32).max(axis=2)
        thr = np.ldexp(1.0, np.maximum(su_o, su_g) - 127 + emax)  # power of two between the two choices
        ok = (np.abs(su_g - su_o) == 1) & (np.abs(amax - thr) <= dblk)
        bad = np.argwhere(diff_s & ~ok)
        assert bad.size == 0, f"{len(bad)} scale bytes differ beyond the boundary rule, first {bad[:4].tolist()}"
        stats["scale_steps"] = int(diff_s.sum())
    same_scale = np.repeat(~diff_s, 32, axis=1)
    # --- elements under equal scales: equal values, or one step across a midpoint within delta
    dv = np.abs(deq_g - deq_o)
    exact = dv == 0
    unit = np.ldexp(1.0, np.repeat(su_o, 32, axis=1) - 127)
    rg = np.abs(deq_g) / unit
    ro = np.abs(deq_o) / unit
    idx_g = np.searchsorted(mags, rg)
    idx_o = np.searchsorted(mags, ro)
    same_sign_or_zero = (np.sign(deq_g) == np.sign(deq_o)) | (deq_g == 0) | (deq_o == 0)
    adjacent = (np.abs(idx_g - idx_o) == 1) & same_sign_or_zero
    mid = 0.5 * (deq_g + deq_o)
    near_mid = np.abs(g32 - mid) <= delta
    ok_elem = exact | (adjacent & near_mid)
    bad = np.argwhere(same_scale & ~ok_elem)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{len(bad)} MX codes differ beyond one step at a midpoint; first {i}: "
                             f"gpu {deq_g[i]!r} oracle {deq_o[i]!r} g {g32[i]!r} delta {delta[i]!r}")
    stats["code_steps"] = int((same_scale & ~exact).sum())
    # --- elements of blocks whose scale legitimately differs: a valid rounding of a value within delta of g
    if diff_s.any():
        unit_g = np.ldexp(1.0, np.repeat(su_g, 32, axis=1) - 127)
        r = np.abs(g32) / unit_g
        spacing = np.ldexp(1.0, np.maximum(O.floor_log2(np.where(r > 0, r, 1.0)), 1 - {"e2m3": 1, "e3m2": 3}[fmt])
                           - {"e2m3": 3, "e3m2": 2}[fmt]) * unit_g
        ok_other = np.abs(deq_g - g32) <= 0.5 * spacing + delta + np.maximum(np.abs(g32) - mags[-1] * unit_g, 0)
        bad = np.argwhere(~same_scale & ~ok_other)
        assert bad.size == 0, f"{len(bad)} codes in scale-flipped blocks are not valid roundings"
    stats["exact"] = int((exact & same_scale).sum())
    return stats


# ---------------------------------------------------------------- 8-bit operands: the instruction's product window

MFMA_WINDOW_BITS = 13


def mfma_window_bound(da: np.ndarray, dw: np.ndarray, block: int = 32) -> np.ndarray:
    """Per-output bound on what the gfx950 scaled MFMA drops from C = A W^T
    when its operands are 8-bit (E4M3 / E5M2).

    Measured on the chip with constructed operands (tests/test_gpu_gemm.py
    pins it): the instruction adds a group of products in a fixed-point
    window whose last bit is 2**(E - 13), E the exponent of the group's
    largest product, truncating each product toward zero onto that grid
    (1 + 2**-13 is kept, 1 + 2**-14 and 1 - 2**-14 come back as 1, and
    1 + 1.5 * 2**-13 as 1 + 2**-13).  Groups never span two 32-element
    blocks, so taking E over the whole block only widens the bound: a product
    loses less than min(|p|, 2**(E_block - 13)), and nothing when it is a
    multiple of 2**(E_block - 13).  The 4- and 6-bit pairs the library runs
    need no such term: for 6-bit operands the instruction's window reaches
    14 binades below its largest product (test_fp6_product_window), every
    E2M3 x E3M2 product is a multiple of 2**-7 and at most 210 < 2**8 (so
    exactly 14 binades), E2M3 x E2M3 products span under 12 binades and
    E2M1 x E2M1 ones 8.  E3M2 x E3M2 products would span 17, which is why
    the library rejects that pair.

    da [M, K], dw [N, K]: dequantized operands (float64).  Returns [M, N]."""
    da = np.asarray(da, dtype=np.float64)
    dw = np.asarray(dw, dtype=np.float64)
    m, k = da.shape
    n = dw.shape[0]
    out = np.zeros((m, n))
    for b in range(k // block):
        p = da[:, None, b * block:(b + 1) * block] * dw[None, :, b * block:(b + 1) * block]  # exact
        a = np.abs(p)
        amax = a.max(axis=2, keepdims=True)
        e = O.floor_log2(np.where(amax > 0, amax, 1.0))  # all-zero blocks lose nothing
        unit = np.ldexp(1.0, e - MFMA_WINDOW_BITS)
        q = a / unit  # exact: a power-of-two division
        lossy = np.floor(q) != q
        out += np.sum(np.where(lossy, np.minimum(a, unit), 0.0), axis=2)
    return out


def assert_close_window(gpu: np.ndarray, c: np.ndarray, s: np.ndarray, wb: np.ndarray, out_kind: str,
                        what: str) -> int:
    """fp32 / bf16 outputs against C with the 8-bit-operand tolerance: the
    GEMM bar (1e-5 * S, or one bf16 ulp) plus the window bound.  Returns how
    many outputs needed the window term."""
    d = np.abs(np.asarray(gpu, dtype=np.float64) - c)
    if out_kind == "f32":
        base = O.GEMM_RTOL * s
        ok = d <= base + wb
    else:
        u = O.ulp_bf16(c)
        base = np.maximum(u, O.GEMM_RTOL * s + 0.5 * u)
        ok = d <= base + wb + 0.5 * O.ulp_bf16(np.abs(c) + wb)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} outputs outside the bound; first {i}: gpu {gpu[i]!r} "
                             f"oracle {c[i]!r} S {s[i]!r} window {wb[i]!r}")
    return int(np.count_nonzero(d > base))


def check_chain_fc2(got: np.ndarray, gpu_h_codes: np.ndarray, gpu_h_scales: np.ndarray, codes_o: np.ndarray,
                    scales_o: np.ndarray, g32: np.ndarray, delta: np.ndarray, dw2: np.ndarray, what: str,
                    fmt: str = "e2m3") -> dict:
    """The second GEMM of an MLP chain, held to the full GEMM bar on every
    checked output.

    1. The GPU's intermediate rows (packed codes and scales, as the first GEMM
       wrote them) must pass the boundary-aware rule against the oracle's
       fp32 intermediate g32 with its allowed distance delta: an element may
       differ from the oracle's code only by one step across a rounding
       midpoint within delta, a scale byte by one at a power of two.
    2. fc2's expected value is the exact product (float64) of that verified
       intermediate with the weights: the oracle's own intermediate plus the
       exact effect of the legitimately different elements.  Every output
       must meet the bf16 bar against it; no fraction of outputs is excused.
    Returns the intermediate's statistics and how many outputs needed the
    bf16 cancellation clause."""
    stats = check_mx_values(gpu_h_codes, gpu_h_scales, g32, delta, fmt)
    n = codes_o.shape[1]
    dh_o = O.dequantize(codes_o, scales_o, fmt)
    dh_g = O.dequantize(O.unpack(gpu_h_codes, n, fmt), gpu_h_scales, fmt)
    c2, s2 = O.gemm_ref(dh_o, dw2)
    diff = dh_g - dh_o
    rows = np.nonzero(diff.any(axis=1))[0]
    if rows.size:
        c2[rows] += diff[rows] @ dw2.T          # = dh_g @ dw2.T on those rows, exactly in float64
        s2[rows] = np.abs(dh_g[rows]) @ np.abs(dw2).T
    stats["fc2_second_clause"] = assert_bf16_close(got, c2, s2, what)
    stats["rows_with_flips"] = int(rows.size)
    return stats
