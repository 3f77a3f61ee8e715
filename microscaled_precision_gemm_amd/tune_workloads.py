"""Tune mx_gemm's launch configuration for the workload shapes on this GPU and
save the table:

    python -m microscaled_precision_gemm_amd.tune_workloads OUT.json

The shapes are the DiT MLP (fc1 with the GELU -> E2M3 epilogue, fc2 to
bf16), the same two GEMMs on one GPU's share of the tokens over 8 GPUs (2560
tokens), its SwiGLU variant (gate/up with the SwiGLU -> E2M3 epilogue, down
projection to bf16), the attention projection, and fc1's shape in each
operand format (bf16 out), all on seeded synthetic operands of the workloads'
distributions.  The table shipped with the package (``tuning.SHIPPED_TABLE``)
was written by this script on an MI355X.
"""

from __future__ import annotations

import sys

import torch

from . import binding as mx
from . import synthetic as syn
from .tuning import TuningTable, tune_gemm


def tune_all(table: TuningTable, log=print) -> TuningTable:
    dev = torch.device("cuda:0")

    def show(name, e):
        log(f"{name}: config {e['config']} {e['us']} us (default {e['default_us']} us)")

    fc1, fc2 = syn.WORKLOADS["fc1"], syn.WORKLOADS["fc2"]
    xq = mx.mx_quantize(syn.make_a(fc1).to(dev), "e2m3")
    w1 = mx.mx_quantize(syn.make_w(fc1).to(dev), "e2m3")
    show("fc1 gelu->e2m3", tune_gemm(table, xq, w1, out_kind="mx", epilogue="gelu_tanh"))
    h = mx.mx_gemm(xq, w1, out_kind="mx", epilogue="gelu_tanh")
    w2 = mx.mx_quantize(syn.make_w(fc2).to(dev), "e2m3")
    show("fc2 bf16", tune_gemm(table, h, w2, out_kind="bf16"))
    del h, w2
    for fmt in ("e2m3", "e2m1", "e4m3"):
        a = xq if fmt == "e2m3" else mx.mx_quantize(syn.make_a(fc1).to(dev), fmt)
        w = w1 if fmt == "e2m3" else mx.mx_quantize(syn.make_w(fc1).to(dev), fmt)
        show(f"fc1-shaped {fmt} bf16", tune_gemm(table, a, w, out_kind="bf16"))
        del a, w
    del xq, w1

    s1, s2 = syn.WORKLOADS["sw_fc1"], syn.WORKLOADS["sw_fc2"]
    xq = mx.mx_quantize(syn.make_a(s1).to(dev), "e2m3")
    w1 = mx.mx_quantize(syn.make_w(s1).to(dev), "e2m3")
    show("SwiGLU gate/up", tune_gemm(table, xq, w1, out_kind="mx", epilogue="swiglu"))
    h = mx.mx_gemm(xq, w1, out_kind="mx", epilogue="swiglu")
    w2 = mx.mx_quantize(syn.make_w(s2).to(dev), "e2m3")
    show("SwiGLU down", tune_gemm(table, h, w2, out_kind="bf16"))
    del xq, w1, h, w2

    # one GPU's share of the 20480 tokens over 8 GPUs (sequence parallelism)
    xq = mx.mx_quantize(syn.make_a(fc1, m=2560).to(dev), "e2m3")
    w1 = mx.mx_quantize(syn.make_w(fc1).to(dev), "e2m3")
    show("fc1 share of 8 GPUs", tune_gemm(table, xq, w1, out_kind="mx", epilogue="gelu_tanh"))
    h = mx.mx_gemm(xq, w1, out_kind="mx", epilogue="gelu_tanh")
    w2 = mx.mx_quantize(syn.make_w(fc2).to(dev), "e2m3")
    show("fc2 share of 8 GPUs", tune_gemm(table, h, w2, out_kind="bf16"))
    del xq, w1, h, w2

    p = syn.WORKLOADS["proj"]
    a = mx.mx_quantize(syn.make_a(p).to(dev), "e2m3")
    w = mx.mx_quantize(syn.make_w(p).to(dev), p.w_fmt)
    show("proj bf16", tune_gemm(table, a, w, out_kind="bf16"))
    return table


def main(argv: list[str]) -> int:
    if len(argv) != 1:
        print(__doc__)
        return 2
    table = tune_all(TuningTable())
    print(f"saved {table.save(argv[0])}")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
