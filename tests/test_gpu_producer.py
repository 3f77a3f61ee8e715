"""mx_rmsnorm_quantize (RMSNorm + modulation + MX quantization into the tiled
GEMM operand layout) on the GPU against the oracle.

The device evaluates the norm in fp32, so its codes are compared with the
oracle's quantization of fp32(y_exact) under the boundary-aware rule: a code
may be one step off only where y lies within the fp32 evaluation bound of a
rounding midpoint, a scale byte may be one off only where the block amax lies
that close to a power of two, and at least 99.9 % of the codes must be exact.
"""

import numpy as np
import pytest
import torch

import microscaled_precision_gemm_amd as mx
from microscaled_precision_gemm_amd import synthetic as syn
from oracle import mx_oracle as O
from tests.parity import check_mx_values, mx_rows_view, rmsnorm_bound, say

pytestmark = pytest.mark.gpu


def _inputs(rows, d, n_cond, seed, src="bf16", modulated=True, with_gamma=True):
    rng = np.random.default_rng([90, seed])
    x = rng.standard_normal((rows, d)).astype(np.float32) * np.exp2(rng.integers(-3, 4, (rows, 1))).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16 if src == "bf16" else torch.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32) if with_gamma else None
    shift = (0.5 * rng.standard_normal((n_cond, d))).astype(np.float32) if modulated else None
    scale = (0.3 * rng.standard_normal((n_cond, d))).astype(np.float32) if modulated else None
    return xt, gamma, shift, scale


def _check(hq, xt, gamma, shift, scale, per, eps, fmt):
    x64 = xt.to(torch.float64).numpy()
    y = O.rmsnorm_modulate(x64, gamma, shift, scale, per, eps)
    y32 = y.astype(np.float32).astype(np.float64)
    gc, gs = mx_rows_view(hq)
    stats = check_mx_values(gc, gs, y32, rmsnorm_bound(x64, gamma, scale, per, eps, y32), fmt)
    assert stats["exact"] >= 0.999 * stats["elements"], stats
    return stats


def _t(v):
    return None if v is None else torch.from_numpy(v).cuda()


@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
@pytest.mark.parametrize("rows,d,per", [(300, 416, 64), (37, 96, 32), (64, 3072, 32), (96, 1024, 96)])
def test_producer_small(src, fmt, rows, d, per):
    n_cond = -(-rows // per)
    xt, gamma, shift, scale = _inputs(rows, d, n_cond, rows + d, src)
    say(f"producer {src} {fmt} {rows}x{d} per={per}")
    hq = mx.mx_rmsnorm_quantize(xt.cuda(), _t(gamma), _t(shift), _t(scale), per, 1e-6, fmt)
    torch.cuda.synchronize()
    _check(hq, xt, gamma, shift, scale, per, 1e-6, fmt)


@pytest.mark.parametrize("src,rows,d", [("f32", 40, 2048), ("bf16", 64, 4096), ("bf16", 40, 5120),
                                         ("f32", 40, 8192)])
def test_producer_row_lengths(src, rows, d):
    """Longer rows than the workloads' (up to 8192 fp32 elements, 32 KB per
    row), bf16 and fp32 sources, a ragged row count."""
    xt, gamma, shift, scale = _inputs(rows, d, 2, d, src)
    say(f"producer {src} {rows}x{d}")
    hq = mx.mx_rmsnorm_quantize(xt.cuda(), _t(gamma), _t(shift), _t(scale), 32, 1e-6, "e2m3")
    torch.cuda.synchronize()
    _check(hq, xt, gamma, shift, scale, 32, 1e-6, "e2m3")


def test_producer_unaligned_parameter_vectors():
    """gamma / shift / scale only 4-byte aligned (views one float into a buffer)."""
    rows, d = 96, 512
    xt, gamma, shift, scale = _inputs(rows, d, 3, 11, "bf16")
    gbuf = torch.zeros(d + 1, dtype=torch.float32)
    gbuf[1:] = torch.from_numpy(gamma)
    sbuf = torch.zeros(3 * d + 1, dtype=torch.float32)
    sbuf[1:] = torch.from_numpy(scale).reshape(-1)
    hbuf = torch.zeros(3 * d + 1, dtype=torch.float32)
    hbuf[1:] = torch.from_numpy(shift).reshape(-1)
    g_, s_, h_ = gbuf.cuda()[1:], sbuf.cuda()[1:].view(3, d), hbuf.cuda()[1:].view(3, d)
    assert g_.data_ptr() % 16 == 4
    say("producer unaligned parameters")
    hq = mx.mx_rmsnorm_quantize(xt.cuda(), g_, h_, s_, 32, 1e-6, "e2m3")
    torch.cuda.synchronize()
    _check(hq, xt, gamma, shift, scale, 32, 1e-6, "e2m3")


@pytest.mark.parametrize("with_gamma", [True, False])
def test_producer_without_modulation(with_gamma):
    """No shift / scale: the plain RMSNorm (with or without a gain) quantized."""
    xt, gamma, _, _ = _inputs(130, 512, 1, 5, "bf16", modulated=False, with_gamma=with_gamma)
    say(f"producer plain norm gamma={with_gamma}")
    hq = mx.mx_rmsnorm_quantize(xt.cuda(), _t(gamma), eps=1e-5)
    torch.cuda.synchronize()
    _check(hq, xt, gamma, None, None, None, 1e-5, "e2m3")


def test_producer_edge_rows():
    """An all-zero row (inv = 1/sqrt(eps)), a row of one huge value, and
    a 16-byte-aligned row stride wider than d."""
    rows, d = 40, 256
    x = np.random.default_rng(7).standard_normal((rows, d + 32)).astype(np.float32)
    x[3] = 0.0
    x[5] = 0.0
    x[5, 17] = 3.0e4
    full = torch.from_numpy(x).to(torch.bfloat16)
    xt = full[:, :d]  # strided view: ld = d + 32
    say("producer edge rows")
    hq = mx.mx_rmsnorm_quantize(full.cuda()[:, :d], eps=1e-6)
    torch.cuda.synchronize()
    _check(hq, xt.contiguous(), None, None, None, None, 1e-6, "e2m3")


def test_producer_is_deterministic_and_feeds_the_gemm():
    """Two calls give the same bytes; the output is a valid GEMM operand (the
    GEMM of the produced activations equals the oracle GEMM of the device's
    own codes within the fp32 bound)."""
    rows, d, n = 256, 512, 256
    xt, gamma, shift, scale = _inputs(rows, d, 2, 8, "bf16")
    w = syn.random_like_workload(9, rows, d, n)[1]
    say("producer -> gemm")
    h1 = mx.mx_rmsnorm_quantize(xt.cuda(), _t(gamma), _t(shift), _t(scale), 128)
    h2 = mx.mx_rmsnorm_quantize(xt.cuda(), _t(gamma), _t(shift), _t(scale), 128)
    wq = mx.mx_quantize(w.cuda(), "e2m3")
    c = mx.mx_gemm(h1, wq, out_kind="f32")
    torch.cuda.synchronize()
    assert torch.equal(h1.codes, h2.codes) and torch.equal(h1.scales, h2.scales)
    gc, gs = mx_rows_view(h1)
    da = O.dequantize(O.unpack(gc, d), gs, "e2m3")
    dw = O.dequantize(*O.quantize(w.to(torch.float64).numpy(), "e2m3"), "e2m3")
    ref, s = O.gemm_ref(da, dw)
    assert O.check_fp32(c.cpu().numpy().astype(np.float64), ref, s).all()


def test_producer_full_size():
    """The fc1 input 20480 x 3072 (bf16), gain and two conditionings of 10240
    rows each, in the launch configuration the bench times; sampled rows, all
    of their blocks."""
    w = syn.WORKLOADS["fc1"]
    x = syn.make_a(w)
    rng = np.random.default_rng([91, w.index])
    gamma = (1.0 + 0.1 * rng.standard_normal(w.k)).astype(np.float32)
    shift = (0.5 * rng.standard_normal((2, w.k))).astype(np.float32)
    scale = (0.3 * rng.standard_normal((2, w.k))).astype(np.float32)
    rows = np.unique(np.concatenate([[0, w.m - 1, 10239, 10240], rng.choice(w.m, 60, replace=False)]))
    say(f"producer full size {w.m}x{w.k}")
    hq = mx.mx_rmsnorm_quantize(x.cuda(), _t(gamma), _t(shift), _t(scale), 10240)
    torch.cuda.synchronize()
    gc, gs = mx_rows_view(hq)
    x64 = x[torch.from_numpy(rows)].to(torch.float64).numpy()
    cond_rows = rows // 10240
    y = O.rmsnorm_modulate(x64, gamma, shift[cond_rows], scale[cond_rows], 1, 1e-6)
    y32 = y.astype(np.float32).astype(np.float64)
    bound = rmsnorm_bound(x64, gamma, scale[cond_rows], 1, 1e-6, y32)
    stats = check_mx_values(gc[rows], gs[rows], y32, bound, "e2m3")
    assert stats["exact"] >= 0.999 * stats["elements"], stats


def test_quantize_once_stacked_projection():
    """Quantize once, one projection GEMM: the producer's single quantized
    activation feeds one mx_gemm over the stacked [Wq; Wk; Wv; Wgate] weights.
    Every output column depends only on its own weight row, so each slice of
    the stacked result is bit-identical to the separate GEMM of that
    projection, and the whole matches the oracle GEMM of the produced codes.
    Ragged rows, K and stacked N."""
    rows, d, outs = 300, 416, (160, 160, 96, 224)
    xt, gamma, shift, scale = _inputs(rows, d, 1, 12, "bf16")
    ws = [syn.random_like_workload(20 + i, rows, d, o)[1] for i, o in enumerate(outs)]
    say("producer -> stacked projection")
    a = mx.mx_rmsnorm_quantize(xt.cuda(), _t(gamma), _t(shift), _t(scale), 320)
    w_stack = mx.mx_quantize(torch.cat(ws).cuda(), "e2m3")
    c = mx.mx_gemm(a, w_stack, out_kind="bf16")
    parts = [mx.mx_gemm(a, mx.mx_quantize(w.cuda(), "e2m3"), out_kind="bf16") for w in ws]
    c32 = mx.mx_gemm(a, w_stack, out_kind="f32")
    torch.cuda.synchronize()
    assert tuple(c.shape) == (rows, sum(outs))
    off = 0
    for o, p in zip(outs, parts):
        assert torch.equal(c[:, off:off + o], p)
        off += o
    gc, gs = mx_rows_view(a)
    da = O.dequantize(O.unpack(gc, d), gs, "e2m3")
    dw = O.dequantize(*O.quantize(torch.cat(ws).to(torch.float64).numpy(), "e2m3"), "e2m3")
    ref, s = O.gemm_ref(da, dw)
    assert O.check_fp32(c32.cpu().numpy().astype(np.float64), ref, s).all()
