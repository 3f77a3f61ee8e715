"""Parity at the workloads' full sizes, in the launch configuration bench.py
times.

Activations are quantized to the tiled layout by mx_quantize (or inside the
split-K call, as the skinny bench does), weights are quantized once, then
mx_gemm / mx_gemm_splitk run at the full shape.  The oracle checks a seeded
sample of outputs that it computes one by one: sampled token rows x sampled
output features (whole 32-feature MX blocks for the MX epilogue), from the
sampled rows of A and W only.  MX quantization works per row along K, so a
row subset quantizes exactly as it does inside the full matrix.  The first
and last rows, features and blocks are always in the sample.
"""

import numpy as np
import pytest
import torch

import microscaled_precision_gemm_amd as mx
from microscaled_precision_gemm_amd import synthetic as syn
from oracle import mx_oracle as O
from tests.parity import (assert_bf16_close, assert_close_window, assert_fp32_close, bf16_tensor_to_f64,
                          check_chain_fc2, check_mx_epilogue, mfma_window_bound, mx_epilogue_target, mx_rows_view,
                          say, swiglu_bound, to_np)

pytestmark = pytest.mark.gpu

ROW_SAMPLE = 40
COL_SAMPLE = 384
BLOCK_SAMPLE = 24


def _pick(total: int, count: int, rng: np.random.Generator) -> np.ndarray:
    count = min(count, total)
    return np.unique(np.concatenate([[0, total - 1], rng.choice(total, size=count, replace=False)]))


def _deq_rows(t: torch.Tensor, rows: np.ndarray, fmt: str) -> np.ndarray:
    return O.dequantize(*O.quantize(syn.as_f64(t[torch.from_numpy(rows)]), fmt), fmt)


@pytest.fixture(scope="module")
def fc2_input():
    return syn.make_a(syn.WORKLOADS["fc2"])


def test_tiny_full_fp32():
    """256 x 256 x 256, fp32 out: every output checked, with the activations
    quantized inside the call and pre-quantized."""
    w = syn.WORKLOADS["tiny"]
    a, wt = syn.make_a(w), syn.make_w(w)
    say("workload tiny 256^3 fp32")
    wq = mx.mx_quantize(wt.cuda(), w.w_fmt)
    o_src = mx.mx_gemm(a.cuda(), wq, out_kind="f32")
    o_pre = mx.mx_gemm(mx.mx_quantize(a.cuda(), "e2m3"), wq, out_kind="f32")
    torch.cuda.synchronize()
    all_rows = np.arange(w.m)
    c, s = O.gemm_ref(_deq_rows(a, all_rows, "e2m3"), _deq_rows(wt, np.arange(w.n), w.w_fmt))
    assert torch.equal(o_src, o_pre)
    assert_fp32_close(to_np(o_pre).astype(np.float64), c, s, "tiny")


@pytest.mark.parametrize("name", ["proj", "fc2"])
def test_full_size_bf16_out(name, request):
    """proj (4096 x 3072 x 3072) and fc2 (20480 x 12288 x 3072, heavy-tailed
    activations with outlier channels), bf16 out, sampled outputs; run twice
    to check the result is deterministic."""
    w = syn.WORKLOADS[name]
    a = request.getfixturevalue("fc2_input") if name == "fc2" else syn.make_a(w)
    wt = syn.make_w(w)
    rng = np.random.default_rng([77, w.index])
    rows, cols = _pick(w.m, ROW_SAMPLE, rng), _pick(w.n, COL_SAMPLE, rng)
    say(f"workload {name} {w.m}x{w.k}x{w.n} bf16 out")
    dev = torch.device("cuda:0")
    aq = mx.mx_quantize(a.to(dev), "e2m3")
    wq = mx.mx_quantize(wt.to(dev), w.w_fmt)
    y = torch.empty((w.m, w.n), dtype=torch.bfloat16, device=dev)
    mx.mx_gemm(aq, wq, out_kind="bf16", out=y)
    y2 = mx.mx_gemm(aq, wq, out_kind="bf16")
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "not deterministic"
    got = bf16_tensor_to_f64(y[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)])
    c, s = O.gemm_ref(_deq_rows(a, rows, "e2m3"), _deq_rows(wt, cols, w.w_fmt))
    assert_bf16_close(got, c, s, f"{name} sampled")


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_operand_formats_full_size(fmt):
    """The MXFP4 / MXFP8 GEMM bench.py times: fc1's shape 20480 x 3072 x
    12288, both operands quantized to `fmt`, bf16 out; sampled outputs
    against the oracle (FP8 with the instruction's product-window bound)."""
    w = syn.WORKLOADS["fc1"]
    a, wt = syn.make_a(w), syn.make_w(w)
    rng = np.random.default_rng([79, w.index, len(fmt)])
    rows, cols = _pick(w.m, ROW_SAMPLE, rng), _pick(w.n, COL_SAMPLE, rng)
    say(f"workload fc1-shaped {w.m}x{w.k}x{w.n} {fmt} x {fmt} bf16 out")
    dev = torch.device("cuda:0")
    aq, wq = mx.mx_quantize(a.to(dev), fmt), mx.mx_quantize(wt.to(dev), fmt)
    y = torch.empty((w.m, w.n), dtype=torch.bfloat16, device=dev)
    mx.mx_gemm(aq, wq, out_kind="bf16", out=y)
    torch.cuda.synchronize()
    got = bf16_tensor_to_f64(y[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)])
    da, dw = _deq_rows(a, rows, fmt), _deq_rows(wt, cols, fmt)
    c, s = O.gemm_ref(da, dw)
    if O.element_bits(fmt) == 8:
        assert_close_window(got, c, s, mfma_window_bound(da, dw), "bf16", f"{fmt} sampled")
    else:
        assert_bf16_close(got, c, s, f"{fmt} sampled")


def test_fc1_full_size_gelu_mx():
    """fc1 20480 x 3072 x 12288 with the GELU-tanh -> E2M3 epilogue: sampled
    token rows x sampled whole 32-feature blocks, under the boundary-aware
    rule (one element step at a rounding midpoint, one scale step at a power
    of two, only within the fp32 accumulation and GELU error).  Every tile
    shape the tuner chooses between for this shape gives the same bytes."""
    w = syn.WORKLOADS["fc1"]
    a, wt = syn.make_a(w), syn.make_w(w)
    rng = np.random.default_rng([78, w.index])
    rows = _pick(w.m, ROW_SAMPLE, rng)
    blocks = _pick(w.n // 32, BLOCK_SAMPLE, rng)
    cols = (blocks[:, None] * 32 + np.arange(32)[None, :]).ravel()
    say(f"workload fc1 {w.m}x{w.k}x{w.n} gelu->e2m3")
    dev = torch.device("cuda:0")
    aq = mx.mx_quantize(a.to(dev), "e2m3")
    wq = mx.mx_quantize(wt.to(dev), w.w_fmt)
    h = mx.MXTensor.empty(w.m, w.n, "e2m3", "tiled", dev)
    mx.mx_gemm(aq, wq, out_kind="mx", epilogue="gelu_tanh", out=h)
    for cfg in ((4, 1, 128, 4), (4, 1, 256, 8)):
        h_other = mx.mx_gemm(aq, wq, out_kind="mx", epilogue="gelu_tanh", config=cfg)
        torch.cuda.synchronize()
        assert torch.equal(h.codes, h_other.codes) and torch.equal(h.scales, h_other.scales), cfg
        del h_other
    gc, gs = mx_rows_view(h)
    codes_g = O.unpack(gc[rows], w.n)[:, cols]
    scales_g = gs[rows][:, blocks]
    c, s = O.gemm_ref(_deq_rows(a, rows, "e2m3"), _deq_rows(wt, cols, w.w_fmt))
    stats = check_mx_epilogue(O.pack(codes_g), scales_g, c, s, True, "e2m3")
    assert stats["exact"] >= 0.999 * stats["elements"], stats


def test_mlp_chain_full_size():
    """The bench's whole step (quantize x, fc1 GELU -> E2M3, fc2 bf16) at full
    size.  fc2's output on sampled tokens is checked against the oracle's own
    chain: the oracle computes those tokens' whole E2M3 intermediate itself.
    The GPU's own intermediate on those tokens must pass the boundary-aware
    rule, and every sampled output meets the bf16 bar against the exact
    product of that verified intermediate."""
    fc1, fc2 = syn.WORKLOADS["fc1"], syn.WORKLOADS["fc2"]
    x, w1, w2 = syn.make_a(fc1), syn.make_w(fc1), syn.make_w(fc2)
    rng = np.random.default_rng([79, fc1.index])
    rows = _pick(fc1.m, 12, rng)
    cols = _pick(fc2.n, COL_SAMPLE, rng)
    say("workload MLP chain 20480 tokens")
    dev = torch.device("cuda:0")
    xq = mx.MXTensor.empty(fc1.m, fc1.k, "e2m3", "tiled", dev)
    h = mx.MXTensor.empty(fc1.m, fc1.n, "e2m3", "tiled", dev)
    y = torch.empty((fc1.m, fc1.k), dtype=torch.bfloat16, device=dev)
    w1q, w2q = mx.mx_quantize(w1.to(dev), "e2m3"), mx.mx_quantize(w2.to(dev), "e2m3")
    mx.mx_quantize(x.to(dev), "e2m3", "tiled", out=xq)
    mx.mx_gemm(xq, w1q, out_kind="mx", epilogue="gelu_tanh", out=h)
    mx.mx_gemm(h, w2q, out_kind="bf16", out=y)
    torch.cuda.synchronize()
    got = bf16_tensor_to_f64(y[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)])
    gc, gs = mx_rows_view(h)
    dw1 = _deq_rows(w1, np.arange(fc1.n), "e2m3")
    codes_o, scales_o, c1, s1, _ = O.fc1_gelu_mx_ref(_deq_rows(x, rows, "e2m3"), dw1)
    g32, delta = mx_epilogue_target(c1, s1, True)
    stats = check_chain_fc2(got, gc[rows], gs[rows], codes_o, scales_o, g32, delta, _deq_rows(w2, cols, "e2m3"),
                            "MLP chain fc2")
    print("MLP chain", stats)


@pytest.mark.parametrize("m", [16, 8])
def test_skinny_full_size_splitk(m):
    """M x 16384 x 13312 with E3M2 weights, 16 splits, activations quantized
    inside the call (as the bench runs it): sampled features, all tokens, bf16
    and fp32 outputs; one split must agree with sixteen within the fp32
    bound, and the call must give the bits of the same split-K call on
    activations quantized beforehand (every output)."""
    w = syn.WORKLOADS["skinny"]
    a, wt = syn.make_a(w, m=m), syn.make_w(w)
    rng = np.random.default_rng([80, m])
    cols = _pick(w.n, 512, rng)
    say(f"workload skinny {m}x{w.k}x{w.n} S={w.splits}")
    dev = torch.device("cuda:0")
    wq = mx.mx_quantize(wt.to(dev), w.w_fmt)
    out = torch.empty((m, w.n), dtype=torch.bfloat16, device=dev)
    work = torch.empty(mx.mx_gemm_workspace_size(m, w.n, w.k, True, w.splits), dtype=torch.uint8, device=dev)
    mx.mx_gemm_splitk(a.to(dev), wq, w.splits, out=out, workspace=work)
    o32 = mx.mx_gemm_splitk(a.to(dev), wq, w.splits, out_kind="f32")
    o32_one = mx.mx_gemm_splitk(a.to(dev), wq, 1, out_kind="f32")
    pre = mx.mx_gemm_splitk(mx.mx_quantize(a.to(dev), "e2m3"), wq, w.splits, out_kind="bf16")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), pre.view(torch.int16))
    ci = torch.from_numpy(cols).to(dev)
    c, s = O.gemm_ref(_deq_rows(a, np.arange(m), "e2m3"), _deq_rows(wt, cols, w.w_fmt))
    assert_bf16_close(bf16_tensor_to_f64(out[:, ci]), c, s, "skinny bf16")
    assert_fp32_close(to_np(o32[:, ci]).astype(np.float64), c, s, "skinny f32")
    assert_fp32_close(to_np(o32_one[:, ci]).astype(np.float64), c, s, "skinny f32 one split")


def _swiglu_sample_ref(x, w, rows, feats, h):
    """Oracle SwiGLU of sampled tokens x sampled output features: the gate and
    up rows of those features (stacked order from the oracle), their GEMMs on
    the sampled token rows, silu(gate) * up."""
    gate_rows, up_rows = O.swiglu_rows(h)
    da = _deq_rows(x, rows, "e2m3")
    g, sg = O.gemm_ref(da, _deq_rows(w, gate_rows[feats], "e2m3"))
    u, su = O.gemm_ref(da, _deq_rows(w, up_rows[feats], "e2m3"))
    return O.silu(g) * u, g, u, sg, su


def test_swiglu_fc1_full_size_mx():
    """SwiGLU fc1 20480 x 3072 x 16384 (stacked gate/up, 8192 features) with the
    E2M3 re-quantization: sampled tokens x sampled whole 32-feature blocks under
    the boundary-aware rule."""
    from tests.parity import check_mx_values, swiglu_bound
    w = syn.WORKLOADS["sw_fc1"]
    h = w.n // 2
    x, wt = syn.make_a(w), syn.make_w(w)
    rng = np.random.default_rng([80, w.index])
    rows = _pick(w.m, ROW_SAMPLE, rng)
    blocks = _pick(h // 32, BLOCK_SAMPLE, rng)
    feats = (blocks[:, None] * 32 + np.arange(32)[None, :]).ravel()
    say(f"workload sw_fc1 {w.m}x{w.k}x{w.n} swiglu->e2m3")
    dev = torch.device("cuda:0")
    xq = mx.mx_quantize(x.to(dev), "e2m3")
    wq = mx.mx_quantize(wt.to(dev), "e2m3")
    hq = mx.MXTensor.empty(w.m, h, "e2m3", "tiled", dev)
    mx.mx_gemm(xq, wq, out_kind="mx", epilogue="swiglu", out=hq)
    # 128-row tiles (one gate/up run each) and 8-wave 256-row tiles: the same bytes
    for cfg in ((4, 1, 128, 4), (4, 1, 256, 8)):
        hn = mx.mx_gemm(xq, wq, out_kind="mx", epilogue="swiglu", config=cfg)
        torch.cuda.synchronize()
        assert torch.equal(hq.codes, hn.codes) and torch.equal(hq.scales, hn.scales), cfg
        del hn
    gc, gs = mx_rows_view(hq)
    codes_g = O.unpack(gc[rows], h)[:, feats]
    out, g, u, sg, su = _swiglu_sample_ref(x, wt, rows, feats, h)
    o32 = out.astype(np.float32).astype(np.float64)
    stats = check_mx_values(O.pack(codes_g), gs[rows][:, blocks], o32, swiglu_bound(g, u, sg, su, o32), "e2m3")
    assert stats["exact"] >= 0.999 * stats["elements"], stats


def test_swiglu_mlp_chain_full_size():
    """The SwiGLU MLP step: quantize x, stacked gate/up GEMM with SwiGLU -> E2M3
    (8192 features), down projection to bf16, at full size; sampled tokens of the
    output against the oracle's chain under the same rule as the GELU chain."""
    w1w, w2w = syn.WORKLOADS["sw_fc1"], syn.WORKLOADS["sw_fc2"]
    h = w1w.n // 2
    x, w1, w2 = syn.make_a(w1w), syn.make_w(w1w), syn.make_w(w2w)
    rng = np.random.default_rng([81, w1w.index])
    rows = _pick(w1w.m, 8, rng)
    cols = _pick(w2w.n, COL_SAMPLE, rng)
    say("workload SwiGLU MLP chain 20480 tokens")
    dev = torch.device("cuda:0")
    xq = mx.mx_quantize(x.to(dev), "e2m3")
    w1q, w2q = mx.mx_quantize(w1.to(dev), "e2m3"), mx.mx_quantize(w2.to(dev), "e2m3")
    hq = mx.mx_gemm(xq, w1q, out_kind="mx", epilogue="swiglu")
    y = mx.mx_gemm(hq, w2q, out_kind="bf16")
    torch.cuda.synchronize()
    got = bf16_tensor_to_f64(y[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)])
    gc, gs = mx_rows_view(hq)
    codes_o, scales_o, out, g, u, sg, su = O.fc1_swiglu_mx_ref(_deq_rows(x, rows, "e2m3"),
                                                              _deq_rows(w1, np.arange(w1w.n), "e2m3"))
    o32 = out.astype(np.float32).astype(np.float64)
    stats = check_chain_fc2(got, gc[rows], gs[rows], codes_o, scales_o, o32, swiglu_bound(g, u, sg, su, o32),
                            _deq_rows(w2, cols, "e2m3"), "SwiGLU MLP chain down projection")
    print("SwiGLU MLP chain", stats)
