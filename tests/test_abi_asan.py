"""The C ABI's host code under AddressSanitizer (no GPU).

api.cpp (argument validation, size and workspace arithmetic, configurations,
the launch log) is rebuilt with the sanitizer on its host side only; the
kernels' objects are the regular build's.  tests/abi_from_c.c, built with the
sanitizer as well, drives every entry point through the paths that need no
device, with and without the launch log: no invalid access and no leak.
"""

import os
import shutil
import subprocess

import pytest

from microscaled_precision_gemm_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM_BIN = "/opt/rocm/lib/llvm/bin"
# host side only: the device code of api.cpp (none that runs here) is built as usual
HOST_ASAN = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()

pytestmark = pytest.mark.slow


def _tool(name: str) -> str:
    path = os.path.join(LLVM_BIN, name)
    if not os.path.exists(path):
        path = shutil.which(name)
    if not path:
        pytest.skip(f"{name} not found")
    return path


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(map(str, cmd))}\n{res.stdout}{res.stderr}"
    return res


def test_host_abi_under_address_sanitizer(tmp_path):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    clang, clangxx = _tool("clang"), _tool("clang++")
    kernels = [os.path.join(B.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "api.cpp"]
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        pytest.skip(f"the library's objects are not built ({os.path.basename(missing[0])})")

    api_o = tmp_path / "api.o"
    flags = [f for f in B.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    _run([hipcc, "-x", "hip", *flags, *HOST_ASAN, "-I", os.path.join(ROOT, "include"), "-I", B.CSRC, "-c",
          os.path.join(B.CSRC, "api.cpp"), "-o", str(api_o)])
    lib = tmp_path / "libmxgemm.so"
    _run([clangxx, "-shared", "-fPIC", "-fsanitize=address", "-o", str(lib), str(api_o), *kernels,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    # the sanitizer really is in the host code: instrumented accesses call its report hooks
    undefined = _run(["nm", "-u", str(lib)]).stdout
    assert "__asan_report_" in undefined

    exe = tmp_path / "abi_from_c"
    _run([clang, "-std=c99", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "abi_from_c.c"),
          "-L", str(tmp_path), "-lmxgemm", f"-Wl,-rpath,{tmp_path}", "-o", str(exe)])
    for log in ("0", "1"):
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", MXGEMM_LOG=log)
        res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
        assert "AddressSanitizer" not in res.stderr, res.stderr
        assert res.returncode == 0, res.stdout + res.stderr
        assert res.stdout.count("ok  ") == 16, res.stdout
        if log == "1":
            assert "mxgemm: mx_gemm " in res.stderr, res.stderr
