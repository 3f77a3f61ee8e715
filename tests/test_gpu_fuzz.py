"""Randomized shapes, deterministic: a seeded draw of GEMM, split-K,
quantizer and producer calls over ragged sizes, every element format pair, output kind,
epilogue and launch configuration the library accepts, each checked against
the oracle at the bar of its kind.  The draw is fixed at import (the test
ids name each case), so a failure reproduces by its id.

Bars: quantizer codes and scales bit-exact; fp32 within 1e-5 * S; bf16 the
two-clause rule; 8-bit operands plus the instruction's product-window bound;
GELU -> MX and SwiGLU outputs under the boundary-aware rule with at least
99.9 % of the codes exact (100 % of the blocks checked); SwiGLU fp32 within
its propagated bound.
"""

import numpy as np
import pytest
import torch

import microscaled_precision_gemm_amd as mx
from microscaled_precision_gemm_amd import synthetic as syn
from oracle import mx_oracle as O
from tests.parity import (GELU_DERIV_MAX, assert_bf16_close, assert_close_window, assert_fp32_close,
                          assert_mx_equal, check_mx_epilogue, check_mx_values, gelu_eval_slack, mfma_window_bound,
                          mx_rows_view, say, swiglu_bound)

pytestmark = pytest.mark.gpu

SIX = [("e2m3", "e2m3"), ("e2m3", "e3m2"), ("e3m2", "e2m3")]
OTHER = [("e2m1", "e2m1"), ("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")]
CONFIGS_256 = [(4, 1, 256, 4), (8, 1, 256, 4), (2, 0, 256, 4), (4, 1, 256, 8), (16, 1, 256, 8), (1, 0, 256, 8)]
CONFIGS_128 = [(4, 1, 128, 4), (8, 0, 128, 4), (16, 1, 128, 4)]


def _draw_gemm_cases(count=80, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        six = rng.random() < 0.7
        a_fmt, w_fmt = (SIX if six else OTHER)[rng.integers(0, 3 if six else 5)]
        if six:
            epi = ["none", "gelu_tanh", "swiglu"][rng.integers(0, 3)]
            out = ["f32", "bf16", "mx"][rng.integers(0, 3)]
            if epi == "gelu_tanh" and out == "bf16":
                out = "mx"
        else:
            epi, out = "none", ["f32", "bf16"][rng.integers(0, 2)]
        m = int(rng.integers(1, 700))
        k = int(32 * rng.integers(1, 33))
        if epi == "swiglu":
            n = int(128 * rng.integers(1, 6))
        elif out == "mx":
            n = int(32 * rng.integers(1, 22))
        else:
            n = int(rng.integers(1, 700))
        cfgs = CONFIGS_256 + (CONFIGS_128 if six else [])
        cfg = None if rng.random() < 0.25 else cfgs[rng.integers(0, len(cfgs))]
        src = bool(rng.random() < 0.5)  # activations quantized inside the call
        out_fmt = ["e2m3", "e3m2"][rng.integers(0, 2)]
        cases.append((i, a_fmt, w_fmt, epi, out, out_fmt, m, n, k, cfg, src))
    return cases


GEMM_CASES = _draw_gemm_cases()


@pytest.mark.parametrize("case", GEMM_CASES,
                         ids=[f"{c[0]}-{c[1]}x{c[2]}-{c[3]}-{c[4]}-{c[6]}x{c[7]}x{c[8]}-{c[9]}" for c in GEMM_CASES])
def test_random_gemm(case):
    i, a_fmt, w_fmt, epi, out, out_fmt, m, n, k, cfg, src = case
    say(f"fuzz gemm {case}")
    a, w = syn.random_like_workload(3000 + i, m, k, n, a_std=1.0, w_std=0.1)
    qa = O.quantize(syn.as_f64(a), a_fmt)
    qw = O.quantize(syn.as_f64(w), w_fmt)
    da, dw = O.dequantize(*qa, a_fmt), O.dequantize(*qw, w_fmt)
    wq = mx.mx_quantize(w.cuda(), w_fmt)
    aq = mx.mx_quantize(a.cuda(), a_fmt)
    a_arg = a.cuda() if src else aq
    res = mx.mx_gemm(a_arg, wq, out_kind=out, epilogue=epi, out_fmt=out_fmt, a_fmt=a_fmt, config=cfg)
    ref = mx.mx_gemm(aq, wq, out_kind=out, epilogue=epi, out_fmt=out_fmt, config=(4, 1, 256, 4))
    torch.cuda.synchronize()
    assert_mx_equal(aq, qa[0], qa[1], "activations")
    assert_mx_equal(wq, qw[0], qw[1], "weights")
    # every configuration and activation form gives the generic configuration's bytes
    if out == "mx":
        assert torch.equal(res.codes, ref.codes) and torch.equal(res.scales, ref.scales)
    else:
        assert torch.equal(res, ref)
    if epi == "swiglu":
        o64, gate, up, sg, su = O.swiglu_ref(da, dw)
        if out == "mx":
            gc, gs = mx_rows_view(res)
            o32 = o64.astype(np.float32).astype(np.float64)
            stats = check_mx_values(gc, gs, o32, swiglu_bound(gate, up, sg, su, o32), out_fmt)
            assert stats["exact"] >= 0.999 * stats["elements"], stats
        else:
            got = res.float().cpu().numpy().astype(np.float64)
            bound = swiglu_bound(gate, up, sg, su, o64) + (O.ulp_bf16(o64) if out == "bf16" else 0.0)
            bad = np.argwhere(np.abs(got - o64) > bound)
            assert bad.size == 0, f"{len(bad)} SwiGLU outputs off; first {bad[0].tolist()}"
        return
    c, s = O.gemm_ref(da, dw)
    if out == "mx":
        gc, gs = mx_rows_view(res)
        stats = check_mx_epilogue(gc, gs, c, s, epi == "gelu_tanh", out_fmt)
        assert stats["exact"] >= 0.999 * stats["elements"], stats
        return
    got = res.float().cpu().numpy().astype(np.float64)
    if epi == "gelu_tanh":  # fp32 out
        g = O.gelu_tanh(c)
        bound = GELU_DERIV_MAX * O.GEMM_RTOL * s + gelu_eval_slack(c, g)
        bad = np.argwhere(np.abs(got - g) > bound)
        assert bad.size == 0, f"{len(bad)} GELU outputs off; first {bad[0].tolist()}"
    elif O.element_bits(a_fmt) == 8:
        assert_close_window(got, c, s, mfma_window_bound(da, dw), out, "fuzz fp8")
    elif out == "f32":
        assert_fp32_close(got, c, s, "fuzz f32")
    else:
        assert_bf16_close(got, c, s, "fuzz bf16")


def _draw_splitk_cases(count=24, seed=2025):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        a_fmt, w_fmt = SIX[rng.integers(0, 3)]
        splits = int([1, 2, 3, 4, 6, 8, 12, 16][rng.integers(0, 8)])
        k = int(128 * splits * rng.integers(1, 5))
        m = int(rng.integers(1, 17))
        n = int(rng.integers(1, 1200))
        out = ["f32", "bf16"][rng.integers(0, 2)]
        src = bool(rng.random() < 0.5)
        cases.append((i, a_fmt, w_fmt, m, n, k, splits, out, src))
    return cases


SPLITK_CASES = _draw_splitk_cases()


@pytest.mark.parametrize("case", SPLITK_CASES,
                         ids=[f"{c[0]}-{c[1]}x{c[2]}-{c[3]}x{c[4]}x{c[5]}-S{c[6]}-{c[7]}" for c in SPLITK_CASES])
def test_random_splitk(case):
    i, a_fmt, w_fmt, m, n, k, splits, out, src = case
    say(f"fuzz split-K {case}")
    a, w = syn.random_like_workload(4000 + i, m, k, n)
    qa = O.quantize(syn.as_f64(a), a_fmt)
    qw = O.quantize(syn.as_f64(w), w_fmt)
    wq = mx.mx_quantize(w.cuda(), w_fmt)
    a_arg = a.cuda() if src else mx.mx_quantize(a.cuda(), a_fmt)
    res = mx.mx_gemm_splitk(a_arg, wq, splits, out_kind=out, a_fmt=a_fmt)
    torch.cuda.synchronize()
    c, s = O.gemm_ref(O.dequantize(*qa, a_fmt), O.dequantize(*qw, w_fmt))
    got = res.float().cpu().numpy().astype(np.float64)
    if out == "f32":
        assert_fp32_close(got, c, s, "fuzz split-K f32")
    else:
        assert_bf16_close(got, c, s, "fuzz split-K bf16")


def _draw_quantize_cases(count=24, seed=2026):
    rng = np.random.default_rng(seed)
    fmts = ["e2m3", "e3m2", "e2m1", "e4m3", "e5m2"]
    cases = []
    for i in range(count):
        rows = int(rng.integers(1, 400))
        k = int(32 * rng.integers(1, 70))
        pad = int(8 * rng.integers(0, 4))  # row stride beyond k, in elements (16-byte steps for bf16)
        cases.append((i, fmts[rng.integers(0, 5)], ["rows", "tiled"][rng.integers(0, 2)],
                      ["bf16", "f32"][rng.integers(0, 2)], rows, k, pad))
    return cases


QUANTIZE_CASES = _draw_quantize_cases()


@pytest.mark.parametrize("case", QUANTIZE_CASES,
                         ids=[f"{c[0]}-{c[1]}-{c[2]}-{c[3]}-{c[4]}x{c[5]}+{c[6]}" for c in QUANTIZE_CASES])
def test_random_quantize(case):
    i, fmt, layout, src, rows, k, pad = case
    say(f"fuzz quantize {case}")
    rng = np.random.default_rng([5000, i])
    x = (rng.standard_normal((rows, k + pad)) * np.exp2(rng.integers(-20, 20, (rows, 1)))).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16 if src == "bf16" else torch.float32)
    view = xt.cuda()[:, :k]  # row stride k + pad elements: a multiple of 16 bytes
    q = mx.mx_quantize(view, fmt, layout)
    torch.cuda.synchronize()
    codes, scales = O.quantize(xt[:, :k].to(torch.float64).numpy(), fmt)
    assert_mx_equal(q, codes, scales, f"quantize {case}")


def _draw_producer_cases(count=16, seed=2027):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        rows = int(rng.integers(1, 300))
        # half up to 3072 (bf16 rows stay in registers), half up to 6368 (the two-pass kernel)
        d = int(32 * rng.integers(1, 97 if rng.random() < 0.5 else 200))
        per = int(32 * rng.integers(1, 5)) if rng.random() < 0.7 else 0  # 0: no modulation
        cases.append((i, ["bf16", "f32"][rng.integers(0, 2)], ["e2m3", "e3m2"][rng.integers(0, 2)], rows, d, per,
                      bool(rng.random() < 0.7), int(8 * rng.integers(0, 3))))
    return cases


PRODUCER_CASES = _draw_producer_cases()


@pytest.mark.parametrize("case", PRODUCER_CASES,
                         ids=[f"{c[0]}-{c[1]}-{c[2]}-{c[3]}x{c[4]}-per{c[5]}-g{int(c[6])}+{c[7]}" for c in PRODUCER_CASES])
def test_random_producer(case):
    from tests.parity import rmsnorm_bound
    i, src, fmt, rows, d, per, with_gamma, pad = case
    say(f"fuzz producer {case}")
    rng = np.random.default_rng([6000, i])
    x = (rng.standard_normal((rows, d + pad)) * np.exp2(rng.integers(-6, 7, (rows, 1)))).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16 if src == "bf16" else torch.float32)
    n_cond = -(-rows // per) if per else 0
    gamma = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32) if with_gamma else None
    shift = (0.5 * rng.standard_normal((n_cond, d))).astype(np.float32) if per else None
    scale = (0.3 * rng.standard_normal((n_cond, d))).astype(np.float32) if per else None
    dev = lambda v: None if v is None else torch.from_numpy(v).cuda()  # noqa: E731
    hq = mx.mx_rmsnorm_quantize(xt.cuda()[:, :d], dev(gamma), dev(shift), dev(scale), per, 1e-6, fmt)
    torch.cuda.synchronize()
    x64 = xt[:, :d].to(torch.float64).numpy()
    y = O.rmsnorm_modulate(x64, gamma, shift, scale, per if per else None, 1e-6)
    y32 = y.astype(np.float32).astype(np.float64)
    gc, gs = mx_rows_view(hq)
    stats = check_mx_values(gc, gs, y32, rmsnorm_bound(x64, gamma, scale, per if per else None, 1e-6, y32), fmt)
    assert stats["exact"] >= 0.999 * stats["elements"], stats
