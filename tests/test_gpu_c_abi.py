"""The hot path driven from a plain C99 program (tests/abi_from_c_gpu.c): no
Python or torch in that process, device memory from hipMalloc, the library's
calls on a HIP stream.  The program runs as a child process; its fp32 results
are checked here against the oracle within 1e-5 * S."""

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from microscaled_precision_gemm_amd import binding as B
from microscaled_precision_gemm_amd import synthetic as syn
from oracle import mx_oracle as O
from tests.parity import assert_fp32_close, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_gemm_and_splitk(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "abi_from_c_gpu"
    lib_dir = os.path.dirname(B.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "abi_from_c_gpu.c"), "-L", lib_dir, "-lmxgemm",
           "-L", "/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{lib_dir}", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    m, n, k = 300, 544, 1024  # ragged M and N; K = 2 x 4 splits x 128
    a, w = syn.random_like_workload(77, m, k, n)
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([m, n, k], dtype=np.int32).tobytes())
        f.write(a.view(torch.int16).numpy().tobytes())
        f.write(w.view(torch.int16).numpy().tobytes())
    say(f"C program: quantize + mx_gemm {m}x{k}x{n} + split-K 16 rows, S=4")
    run = subprocess.run([str(exe), str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    got = np.fromfile(out, dtype=np.float32)
    assert got.size == m * n + 16 * n
    c, s = O.gemm_ref(O.dequantize(*O.quantize(syn.as_f64(a), "e2m3"), "e2m3"),
                      O.dequantize(*O.quantize(syn.as_f64(w), "e2m3"), "e2m3"))
    assert_fp32_close(got[:m * n].reshape(m, n).astype(np.float64), c, s, "C program mx_gemm")
    assert_fp32_close(got[m * n:].reshape(16, n).astype(np.float64), c[:16], s[:16], "C program mx_gemm_splitk")
