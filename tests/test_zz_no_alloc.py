"""mx_gemm_splitk_noalloc (the allocation-free split-K entry point) against
mx_gemm_splitk on the GPU, through the C ABI: the same bytes on two calls in
a row, the second with a smaller input, so that the static scratch keeps the
first call's larger contents when the second one runs."""

import numpy as np
import pytest
import torch

import microscaled_precision_gemm_amd as mx
from microscaled_precision_gemm_amd import synthetic as syn
from oracle import mx_oracle as O
from tests.parity import assert_bf16_close, assert_fp32_close, bf16_tensor_to_f64, say, to_np

pytestmark = pytest.mark.gpu


def _case(m, n, k, splits, w_fmt, seed, out_kind):
    a, w = syn.random_like_workload(seed, m, k, n, a_std=1.0, w_std=0.02)
    dev = torch.device("cuda:0")
    wq = mx.mx_quantize(w.to(dev), w_fmt)
    ref = mx.mx_gemm_splitk(a.to(dev), wq, splits, out_kind=out_kind)
    dtype = torch.float32 if out_kind == "f32" else torch.bfloat16
    out = torch.full((m, n), float("nan"), dtype=dtype, device=dev)
    mx.mx_gemm_splitk(a.to(dev), wq, splits, out_kind=out_kind, out=out, noalloc=True)
    return a, w, ref, out


@pytest.mark.parametrize("out_kind", ["bf16", "f32"])
def test_noalloc_matches_splitk_twice_second_smaller(out_kind):
    torch.cuda.synchronize()
    results = []
    # first call: 16 tokens, K = 16384 (the skinny workload's K), 13312 features
    # in the full run's layout would be heavy here; 2048 features keep it quick
    for (m, n, k, splits, seed) in ((16, 2048, 16384, 16, 1), (5, 1056, 4096, 8, 2)):
        say(f"noalloc split-K {m}x{n}x{k} S={splits} {out_kind}")
        a, w, ref, out = _case(m, n, k, splits, "e3m2", seed, out_kind)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{m}x{n}x{k}: noalloc differs from mx_gemm_splitk"
        results.append((a, w, out))
    # and both against the oracle on sampled features
    for a, w, out in results:
        m, k = a.shape
        cols = np.unique(np.r_[0, w.shape[0] - 1, np.random.default_rng(5).choice(w.shape[0], 256, replace=False)])
        da = O.dequantize(*O.quantize(syn.as_f64(a), "e2m3"), "e2m3")
        dw = O.dequantize(*O.quantize(syn.as_f64(w[torch.from_numpy(cols)]), "e3m2"), "e3m2")
        c, s = O.gemm_ref(da, dw)
        got = out[:, torch.from_numpy(cols).cuda()]
        if out_kind == "f32":
            assert_fp32_close(to_np(got).astype(np.float64), c, s, "noalloc f32")
        else:
            assert_bf16_close(bf16_tensor_to_f64(got), c, s, "noalloc bf16")


def test_noalloc_pre_quantized_and_limits():
    """Pre-quantized activations need no scratch; K beyond the scratch is
    refused with MX_ERR_SCRATCH before anything runs."""
    dev = torch.device("cuda:0")
    a, w = syn.random_like_workload(3, 8, 1024, 512, a_std=1.0, w_std=0.02)
    wq = mx.mx_quantize(w.to(dev), "e2m3")
    aq = mx.mx_quantize(a.to(dev), "e2m3")
    say("noalloc split-K pre-quantized 8x512x1024")
    ref = mx.mx_gemm_splitk(aq, wq, 4, out_kind="f32")
    out = torch.empty((8, 512), dtype=torch.float32, device=dev)
    mx.mx_gemm_splitk(aq, wq, 4, out_kind="f32", out=out, noalloc=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    big_k = mx.binding.MX_NOALLOC_MAX_K + 2048
    a_big = torch.zeros((2, big_k), dtype=torch.bfloat16, device=dev)
    w_big = mx.MXTensor.empty(32, big_k, "e2m3", "tiled", dev)
    with pytest.raises(mx.binding.MXError) as e:
        mx.mx_gemm_splitk(a_big, w_big, 2, out_kind="f32", out=torch.empty((2, 32), device=dev), noalloc=True)
    assert e.value.status == mx.binding.MX_ERR_SCRATCH
