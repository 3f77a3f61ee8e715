"""Streams and graph capture: every call is asynchronous on the stream it is
given and keeps no state between calls (the allocation-free split-K entry
point aside, whose static scratch is per GPU), so

* the same work on two streams at once gives the bytes of a serial run;
* the hot path captured into a HIP graph (torch.cuda.CUDAGraph) and replayed
  gives the eager bytes on every replay, with eager work on the same buffers'
  inputs between the replays.

Streams keep the default priority.  Nothing here clears memory inside a
captured graph: the kernels write every byte they own.
"""

import numpy as np
import pytest
import torch

import microscaled_precision_gemm_amd as mx
from microscaled_precision_gemm_amd import synthetic as syn
from tests.parity import say

pytestmark = pytest.mark.gpu

M, D, H = 1000, 1024, 2048  # tokens (ragged: not a multiple of 256), model width, hidden width


def _mlp_inputs(seed):
    x, w1 = syn.random_like_workload(seed, M, D, H)
    _, w2 = syn.random_like_workload(seed + 1, 1, H, D)
    dev = torch.device("cuda:0")
    return x.to(dev), mx.mx_quantize(w1.to(dev), "e2m3"), mx.mx_quantize(w2.to(dev), "e2m3")


def _mlp(x, w1, w2, xq=None, h=None, y=None):
    """quantize x -> fc1 GELU -> E2M3 -> fc2 bf16, into the given buffers (or new ones)."""
    xq = mx.mx_quantize(x, "e2m3", out=xq)
    h = mx.mx_gemm(xq, w1, out_kind="mx", epilogue="gelu_tanh", out=h)
    return mx.mx_gemm(h, w2, out_kind="bf16", out=y)


def _same_mx(a, b):
    return torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)


def test_two_streams_match_serial():
    """Two MLP passes and two split-K calls (each with its own workspace)
    enqueued on two streams at once give the serial run's bytes."""
    say("two streams")
    ins = [_mlp_inputs(60), _mlp_inputs(70)]
    a16 = [syn.random_like_workload(80 + i, 16, 4096, 1)[0].cuda() for i in range(2)]
    wsk = mx.mx_quantize(syn.random_like_workload(90, 1, 4096, 1536)[1].cuda(), "e3m2")
    ref = [_mlp(*i) for i in ins]
    ref_sk = [mx.mx_gemm_splitk(a, wsk, 8, out_kind="f32") for a in a16]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs, outs_sk = [None, None], [None, None]
    for rep in range(3):
        torch.cuda.synchronize()
        for s_i, s in enumerate(streams):
            with torch.cuda.stream(s):
                outs[s_i] = _mlp(*ins[s_i])
                outs_sk[s_i] = mx.mx_gemm_splitk(a16[s_i], wsk, 8, out_kind="f32")
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], ref[i]), (rep, i)
            assert torch.equal(outs_sk[i], ref_sk[i]), (rep, i)


def test_graph_replay_matches_eager():
    """quantize -> fc1 (GELU -> E2M3) -> fc2 and the skinny split-K (both the
    workspace and the allocation-free entry point) captured once and replayed
    four times; the inputs are rewritten eagerly between replays and every
    replay must equal the eager result for the inputs it saw."""
    say("graph capture")
    x, w1, w2 = _mlp_inputs(100)
    dev = x.device
    xq = mx.MXTensor.empty(M, D, "e2m3", "tiled", dev)
    h = mx.MXTensor.empty(M, H, "e2m3", "tiled", dev)
    y = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    a16 = syn.random_like_workload(101, 16, 4096, 1)[0].cuda()
    wsk = mx.mx_quantize(syn.random_like_workload(102, 1, 4096, 1536)[1].cuda(), "e3m2")
    ws = torch.empty(mx.mx_gemm_workspace_size(16, 1536, 4096, True, 8), dtype=torch.uint8, device=dev)
    ysk = torch.empty((16, 1536), dtype=torch.float32, device=dev)
    ysk_na = torch.empty((16, 1536), dtype=torch.float32, device=dev)

    def step():
        _mlp(x, w1, w2, xq, h, y)
        mx.mx_gemm_splitk(a16, wsk, 8, out_kind="f32", out=ysk, workspace=ws)
        mx.mx_gemm_splitk(a16, wsk, 8, out_kind="f32", out=ysk_na, noalloc=True)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up outside the capture (the allocation-free path looks up its scratch here)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(103)
    for rep in range(4):
        # new inputs, written eagerly into the captured input buffers
        x.copy_(torch.randn(M, D, generator=gen).to(torch.bfloat16))
        a16.copy_(torch.randn(16, 4096, generator=gen).to(torch.bfloat16))
        want_y = _mlp(x, w1, w2)
        want_h = mx.mx_gemm(mx.mx_quantize(x, "e2m3"), w1, out_kind="mx", epilogue="gelu_tanh")
        want_sk = mx.mx_gemm_splitk(a16, wsk, 8, out_kind="f32")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same_mx(h, want_h), rep
        assert torch.equal(y, want_y), rep
        assert torch.equal(ysk, want_sk) and torch.equal(ysk_na, want_sk), rep
        assert not torch.equal(y, torch.zeros_like(y))
    del g
    np.testing.assert_array_equal(ysk.cpu().numpy(), ysk_na.cpu().numpy())
