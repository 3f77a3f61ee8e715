"""Buffers beyond 4 GiB: every kernel of the path on operands, outputs or
weights whose byte offsets pass 2^32, so that an offset computed in 32 bits
anywhere would show as wrong rows at the end of the buffer.

Inputs of many GiB are drawn on the device (synthetic.device_normal_bf16,
seeded); the oracle sees the sampled rows read back from there.  Sampled rows
always include the last one, whose bytes in the tiled layout lie past 4 GiB in
its later stages, and the tiled codes of the sampled rows are gathered on the
device (tests.parity.mx_rows_gather), so only their bytes cross to the host.
"""

import numpy as np
import pytest
import torch

import microscaled_precision_gemm_amd as mx
from microscaled_precision_gemm_amd import synthetic as syn
from oracle import mx_oracle as O
from tests.parity import (assert_bf16_close, check_mx_epilogue, check_mx_values, mx_rows_gather, rmsnorm_bound,
                          say, to_np)

pytestmark = pytest.mark.gpu

GIB = 1 << 30


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _need(gib: float) -> None:
    free, _ = torch.cuda.mem_get_info()
    if free < gib * GIB:
        pytest.skip(f"needs {gib} GiB of free device memory, {free / GIB:.1f} GiB free")


def _pick(total: int, count: int, seed: int, always=()) -> np.ndarray:
    rng = np.random.default_rng([97, seed])
    return np.unique(np.concatenate([[0, total - 1, *always], rng.choice(total, size=count, replace=False)]))


def _rows64(t: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    return t[torch.from_numpy(rows).to(t.device)].to(torch.float64).cpu().numpy()


def test_quantize_and_gemm_activations_beyond_4gib():
    """A 65536 x 98304 (12 GiB of bf16, 4.5 GiB of E2M3 codes) times W 256 x
    98304, bf16 out: the quantizer's codes of sampled rows bit-exact, the GEMM's
    sampled rows within the bf16 bar, the in-call quantization identical."""
    _need(30)
    m, k, n = 65536, 98304, 256
    dev = torch.device("cuda:0")
    say(f"large activations {m}x{k}x{n}")
    a = syn.device_normal_bf16(m, k, seed=9101, std=1.0, device=dev)
    aq = mx.mx_quantize(a, "e2m3")
    assert aq.codes.numel() > 1 << 32
    _, wt = syn.random_like_workload(41, 1, k, n)
    wq = mx.mx_quantize(wt.to(dev), "e2m3")
    y = mx.mx_gemm(aq, wq, out_kind="bf16")
    y_src = mx.mx_gemm(a, wq, out_kind="bf16")  # quantized inside the call, into a 6 GiB workspace
    torch.cuda.synchronize()
    assert torch.equal(y, y_src)
    rows = _pick(m, 12, 1, always=(1, 31, 32, m - 33))
    codes_o, scales_o = O.quantize(_rows64(a, rows), "e2m3")
    gc, gs = mx_rows_gather(aq, rows)
    assert np.array_equal(gs, scales_o), "scale bytes differ"
    assert np.array_equal(gc, O.pack(codes_o)), "codes differ"
    dw = O.dequantize(*O.quantize(syn.as_f64(wt), "e2m3"), "e2m3")
    c, s = O.gemm_ref(O.dequantize(codes_o, scales_o, "e2m3"), dw)
    assert_bf16_close(to_np(y[torch.from_numpy(rows).to(dev)].float()).astype(np.float64), c, s, "large A")


def test_gemm_outputs_beyond_4gib():
    """262144 x 256 times W 24576 x 256: a bf16 output of 12 GiB and a GELU ->
    E2M3 output of 4.5 GiB of codes; sampled rows (all their 32-feature blocks
    for the MX output, sampled columns for bf16) against the oracle."""
    _need(24)
    m, k, n = 262144, 256, 24576
    dev = torch.device("cuda:0")
    say(f"large outputs {m}x{k}x{n}")
    a = syn.device_normal_bf16(m, k, seed=9102, std=1.0, device=dev)
    _, wt = syn.random_like_workload(42, 1, k, n, w_std=0.1)
    aq = mx.mx_quantize(a, "e2m3")
    wq = mx.mx_quantize(wt.to(dev), "e2m3")
    h = mx.mx_gemm(aq, wq, out_kind="mx", epilogue="gelu_tanh")
    assert h.codes.numel() > 1 << 32
    rows = _pick(m, 6, 2, always=(m - 256, m - 32))
    torch.cuda.synchronize()
    da = O.dequantize(*O.quantize(_rows64(a, rows), "e2m3"), "e2m3")
    dw = O.dequantize(*O.quantize(syn.as_f64(wt), "e2m3"), "e2m3")
    c, s = O.gemm_ref(da, dw)
    gc, gs = mx_rows_gather(h, rows)
    stats = check_mx_epilogue(gc, gs, c, s, True, "e2m3")
    assert stats["exact"] >= 0.999 * stats["elements"], stats
    del h
    y = mx.mx_gemm(aq, wq, out_kind="bf16")
    assert y.numel() * 2 > 1 << 32
    cols = _pick(n, 500, 3)
    torch.cuda.synchronize()
    yr = to_np(y[torch.from_numpy(rows).to(dev)].float()).astype(np.float64)
    assert_bf16_close(yr[:, cols], c[:, cols], s[:, cols], "large bf16 out")


def test_splitk_weights_beyond_4gib():
    """Split-K with W 65536 x 98304 (12 GiB of bf16, 4.5 GiB of E3M2 codes), 16
    tokens, S = 16, activations quantized inside the call: the weights' codes
    of sampled rows bit-exact, sampled output features within the bf16 bar."""
    _need(24)
    m, k, n = 16, 98304, 65536
    dev = torch.device("cuda:0")
    say(f"large split-K weights {m}x{k}x{n} S=16")
    w = syn.device_normal_bf16(n, k, seed=9103, std=0.02, device=dev)
    wq = mx.mx_quantize(w, "e3m2")
    assert wq.codes.numel() > 1 << 32
    a, _ = syn.random_like_workload(43, m, k, 1)
    y = mx.mx_gemm_splitk(a.to(dev), wq, 16, out_kind="bf16")
    cols = _pick(n, 40, 4, always=(1, 31, 32, n - 33))
    torch.cuda.synchronize()
    w64 = _rows64(w, cols)
    del w
    codes_o, scales_o = O.quantize(w64, "e3m2")
    gc, gs = mx_rows_gather(wq, cols)
    assert np.array_equal(gs, scales_o), "weight scale bytes differ"
    assert np.array_equal(gc, O.pack(codes_o, "e3m2")), "weight codes differ"
    da = O.dequantize(*O.quantize(syn.as_f64(a), "e2m3"), "e2m3")
    c, s = O.gemm_ref(da, O.dequantize(codes_o, scales_o, "e3m2"))
    assert_bf16_close(to_np(y.float())[:, cols].astype(np.float64), c, s, "large split-K")


def test_producer_beyond_4gib():
    """RMSNorm + modulation + quantization of 2^21 x 3072 bf16 rows (12 GiB in,
    4.5 GiB of E2M3 codes out), gain and two conditionings of 2^20 rows each;
    sampled rows, all their blocks, under the boundary-aware rule."""
    _need(20)
    rows, d, per = 1 << 21, 3072, 1 << 20
    dev = torch.device("cuda:0")
    say(f"large producer {rows}x{d}")
    x = syn.device_normal_bf16(rows, d, seed=9104, std=1.0, device=dev)
    rng = np.random.default_rng([97, 5])
    gamma = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    shift = (0.5 * rng.standard_normal((2, d))).astype(np.float32)
    scale = (0.3 * rng.standard_normal((2, d))).astype(np.float32)
    hq = mx.mx_rmsnorm_quantize(x, torch.from_numpy(gamma).to(dev), torch.from_numpy(shift).to(dev),
                                torch.from_numpy(scale).to(dev), per)
    assert hq.codes.numel() > 1 << 32
    pick = _pick(rows, 30, 6, always=(per - 1, per, rows - 33))
    torch.cuda.synchronize()
    x64 = _rows64(x, pick)
    cond = pick // per
    y = O.rmsnorm_modulate(x64, gamma, shift[cond], scale[cond], 1, 1e-6)
    y32 = y.astype(np.float32).astype(np.float64)
    gc, gs = mx_rows_gather(hq, pick)
    stats = check_mx_values(gc, gs, y32, rmsnorm_bound(x64, gamma, scale[cond], 1, 1e-6, y32), "e2m3")
    assert stats["exact"] >= 0.999 * stats["elements"], stats
