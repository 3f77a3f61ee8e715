"""Build libmxgemm.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m microscaled_precision_gemm_amd.build

Objects go to ``microscaled_precision_gemm_amd/_build/``; the shared library
is written next to this file, where the Python binding loads it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libmxgemm.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# measurement only (bench.py): the matrix-instruction rate with nothing else in the loop
PROBE_SOURCE = "mfma_ceiling.hip"
PROBE_PATH = os.path.join(PKG, "libmxprobe.so")

SOURCES = ["api.cpp", "quantize.hip", "gemm_we2m3_e2m3.hip", "gemm_we3m2_e2m3.hip", "gemm_we2m3_e3m2.hip",
           "gemm_we2m1_e2m1.hip", "gemm_wfp8_fp8.hip", "splitk.hip", "producer.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # no packed-fp32 VALU instructions (v_pk_{add,mul,fma}_f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(objs: list[str], path: str) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950, link libmxgemm.so (and the
    measurement probe libmxprobe.so); returns the library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + [PROBE_SOURCE]
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:-1], LIB_PATH)
    _link(objs[-1:], PROBE_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
