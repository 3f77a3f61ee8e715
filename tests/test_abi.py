"""The C ABI library on a host without a GPU: it loads, exports every symbol
that include/mxgemm.h declares, and rejects invalid arguments on the host
before any HIP call (status codes, nothing launched)."""

import ctypes
import os
import re
import subprocess

import pytest

import microscaled_precision_gemm_amd as mx
from microscaled_precision_gemm_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxgemm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libmxgemm.so not built")
    return mx.lib()


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(mx.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mx_[a-z_0-9]+)$", out, flags=re.M))
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_version_and_status_strings(L):
    assert mx.mx_version() == 400
    for st in range(-8, 1):
        assert mx.mx_status_string(st) and mx.mx_status_string(st) != "unknown status"
    assert mx.mx_status_string(-99) == "unknown status"


FAKE = 0x100000  # never dereferenced: every call below fails validation first
NULL = None

try:
    import torch as _torch

    _HAS_GPU = _torch.cuda.is_available()
except Exception:  # pragma: no cover
    _HAS_GPU = False

# The calls below pass made-up device addresses that host validation must
# reject.  They are host-logic tests: run them where no GPU is visible, so a
# validation regression can never turn into a launch on bogus pointers.
host_only = pytest.mark.skipif(_HAS_GPU, reason="fake-pointer validation tests run on GPU-less hosts only")


def q(*a):
    return mx.lib().mx_quantize(*a)


@host_only
def test_quantize_validation(L):
    s = NULL
    assert q(FAKE, 5, 4, 64, 64, 2, 1, FAKE, FAKE, s) == B.MX_ERR_FORMAT
    assert q(FAKE, 0, 4, 64, 64, 7, 1, FAKE, FAKE, s) == B.MX_ERR_FORMAT
    assert q(FAKE, 0, -1, 64, 64, 2, 1, FAKE, FAKE, s) == B.MX_ERR_SHAPE
    assert q(FAKE, 0, 4, 48, 48, 2, 1, FAKE, FAKE, s) == B.MX_ERR_SHAPE
    assert q(FAKE, 0, 4, 64, 32, 2, 1, FAKE, FAKE, s) == B.MX_ERR_SHAPE
    assert q(NULL, 0, 4, 64, 64, 2, 1, FAKE, FAKE, s) == B.MX_ERR_NULL
    assert q(FAKE, 0, 4, 64, 64, 2, 1, NULL, FAKE, s) == B.MX_ERR_NULL
    assert q(FAKE + 2, 0, 4, 64, 64, 2, 1, FAKE, FAKE, s) == B.MX_ERR_ALIGN
    assert q(FAKE, 0, 4, 64, 68, 2, 1, FAKE, FAKE, s) == B.MX_ERR_ALIGN
    assert q(FAKE, 0, 4, 64, 64, 2, 1, FAKE + 4, FAKE, s) == B.MX_ERR_ALIGN
    assert q(FAKE, 0, 4, 64, 64, 2, 7, FAKE, FAKE, s) == B.MX_ERR_FORMAT  # layout
    assert q(FAKE, 0, 4, 64, 64, 2, 0, FAKE, FAKE + 2, s) == B.MX_ERR_ALIGN  # scales
    assert q(NULL, 0, 0, 64, 64, 2, 1, NULL, NULL, s) == B.MX_OK  # empty is a no-op
    assert q(NULL, 0, 4, 0, 0, 2, 1, NULL, NULL, s) == B.MX_OK


def rq(**kw):
    a = dict(x=FAKE, src_type=0, rows=64, d=128, ld=128, gamma=NULL, shift=NULL, scale=NULL, per=0,
             eps=ctypes.c_float(1e-6), fmt=2, codes=FAKE, scales=FAKE, stream=NULL)
    a.update(kw)
    return mx.lib().mx_rmsnorm_quantize(*a.values())


@host_only
def test_rmsnorm_quantize_validation(L):
    assert rq(d=100) == B.MX_ERR_SHAPE
    assert rq(rows=-1) == B.MX_ERR_SHAPE
    assert rq(ld=96) == B.MX_ERR_SHAPE
    assert rq(src_type=5) == B.MX_ERR_FORMAT
    assert rq(fmt=7) == B.MX_ERR_FORMAT
    assert rq(fmt=4) == B.MX_ERR_UNSUPPORTED  # the producer writes the 6-bit types
    assert rq(fmt=0) == B.MX_ERR_UNSUPPORTED
    assert rq(x=NULL) == B.MX_ERR_NULL
    assert rq(codes=NULL) == B.MX_ERR_NULL
    assert rq(x=FAKE + 8) == B.MX_ERR_ALIGN
    assert rq(ld=132) == B.MX_ERR_ALIGN
    assert rq(scales=FAKE + 2) == B.MX_ERR_ALIGN
    assert rq(gamma=FAKE + 2) == B.MX_ERR_ALIGN
    assert rq(eps=ctypes.c_float(-1.0)) == B.MX_ERR_SHAPE
    assert rq(eps=ctypes.c_float(float("nan"))) == B.MX_ERR_SHAPE
    assert rq(eps=ctypes.c_float(float("inf"))) == B.MX_ERR_SHAPE
    # modulation needs a positive multiple of 32 rows per conditioning row
    assert rq(shift=FAKE) == B.MX_ERR_SHAPE
    assert rq(scale=FAKE, per=48) == B.MX_ERR_SHAPE
    assert rq(rows=0) == B.MX_OK and rq(d=0) == B.MX_OK
    assert rq(rows=0, shift=FAKE, per=64) == B.MX_OK


def g(**kw):
    a = dict(a_src=NULL, a_src_type=0, lda=0, a_codes=FAKE, a_scales=FAKE, a_fmt=2, w_codes=FAKE, w_scales=FAKE,
             w_fmt=2, m=64, n=64, k=128, epi=0, out_kind=1, out=FAKE, ldo=64, out_scales=NULL, out_fmt=2,
             ws=NULL, ws_bytes=0, stream=NULL)
    a.update(kw)
    return mx.lib().mx_gemm(*a.values())


@host_only
def test_gemm_validation(L):
    assert g(k=100) == B.MX_ERR_SHAPE
    assert g(m=-1) == B.MX_ERR_SHAPE
    assert g(a_fmt=7) == B.MX_ERR_FORMAT
    assert g(a_fmt=4) == B.MX_ERR_UNSUPPORTED  # E2M1 x E2M3: operands of different widths
    assert g(a_fmt=0, w_fmt=2) == B.MX_ERR_UNSUPPORTED
    # 4- and 8-bit pairs: plain product, fp32 / bf16 output
    assert g(a_fmt=4, w_fmt=4, epi=1) == B.MX_ERR_UNSUPPORTED
    assert g(a_fmt=0, w_fmt=1, out_kind=2, out_scales=FAKE) == B.MX_ERR_UNSUPPORTED
    assert g(a_fmt=4, w_fmt=4, m=0) == B.MX_OK and g(a_fmt=1, w_fmt=0, n=0) == B.MX_OK
    assert g(a_src=FAKE) == B.MX_ERR_NULL  # both activation forms
    assert g(a_codes=NULL) == B.MX_ERR_NULL  # neither
    assert g(a_scales=NULL) == B.MX_ERR_NULL
    assert g(w_scales=NULL) == B.MX_ERR_NULL
    assert g(a_codes=FAKE + 8) == B.MX_ERR_ALIGN
    assert g(w_scales=FAKE + 1) == B.MX_ERR_ALIGN
    assert g(a_fmt=3, w_fmt=3) == B.MX_ERR_UNSUPPORTED
    assert g(epi=5) == B.MX_ERR_FORMAT
    assert g(out_kind=9) == B.MX_ERR_FORMAT
    assert g(out=NULL) == B.MX_ERR_NULL
    assert g(ldo=32) == B.MX_ERR_SHAPE
    assert g(out_kind=2, out_scales=FAKE, n=48) == B.MX_ERR_UNSUPPORTED
    assert g(out_kind=2, out_scales=NULL) == B.MX_ERR_NULL
    assert g(out_kind=2, out_scales=FAKE, out_fmt=9) == B.MX_ERR_FORMAT
    assert g(out_kind=2, out_scales=FAKE, out_fmt=1) == B.MX_ERR_UNSUPPORTED  # MX output in the 6-bit types
    assert g(out_kind=2, out_scales=FAKE, out=FAKE + 4) == B.MX_ERR_ALIGN
    # bf16 activations need a workspace for the quantized copy
    assert g(a_src=FAKE, a_codes=NULL, a_scales=NULL, lda=128) == B.MX_ERR_WORKSPACE
    need = mx.mx_gemm_workspace_size(64, 64, 128, True, 0)
    assert need >= 2 * 4096 + 2 * 128  # 1 stage x 2 row groups, tiled, sized for 8-bit codes
    assert g(a_src=FAKE, a_codes=NULL, a_scales=NULL, lda=128, ws=FAKE, ws_bytes=need - 1) == B.MX_ERR_WORKSPACE
    assert g(a_src=FAKE, a_codes=NULL, a_scales=NULL, lda=120, ws=FAKE, ws_bytes=need) == B.MX_ERR_SHAPE
    assert g(a_src=FAKE, a_codes=NULL, a_scales=NULL, lda=130, ws=FAKE, ws_bytes=need) == B.MX_ERR_ALIGN
    assert g(m=0) == B.MX_OK and g(n=0) == B.MX_OK  # empty is a no-op
    # SwiGLU: stacked gate/up rows come in runs of 128; the output has n / 2 columns
    assert g(epi=2, n=192, ldo=96) == B.MX_ERR_UNSUPPORTED
    assert g(epi=2, n=128, ldo=63) == B.MX_ERR_SHAPE
    assert g(epi=2, n=128, ldo=64, m=0) == B.MX_OK
    assert g(epi=2, n=128, out_kind=2, out_scales=FAKE, m=0) == B.MX_OK


@host_only
def test_gemm_config_validation(L):
    args = dict(a_src=NULL, a_src_type=0, lda=0, a_codes=FAKE, a_scales=FAKE, a_fmt=2, w_codes=FAKE,
                w_scales=FAKE, w_fmt=2, m=64, n=64, k=128, epi=0, out_kind=1, out=FAKE, ldo=64, out_scales=NULL,
                out_fmt=2, ws=NULL, ws_bytes=0)
    d = B.MXGemmConfig()
    L.mx_gemm_default_config(ctypes.byref(d))
    assert d.key() == (4, 1, 256, 4)
    for bad in ((0, 1), (17, 1), (4, 2), (4, -1), (4, 1, 64), (4, 1, 0), (4, 1, 512), (4, 1, 256, 2),
                (4, 1, 256, 16), (4, 1, 256, 0)):
        c = B.MXGemmConfig(*bad)
        assert L.mx_gemm_with_config(*args.values(), ctypes.byref(c), NULL) == B.MX_ERR_FORMAT
    ok = B.MXGemmConfig(8, 0)
    assert L.mx_gemm_with_config(*dict(args, m=0).values(), ctypes.byref(ok), NULL) == B.MX_OK
    assert L.mx_gemm_with_config(*dict(args, k=100).values(), ctypes.byref(ok), NULL) == B.MX_ERR_SHAPE
    # 128-feature tiles: the 6-bit pairs (every epilogue); other pairs are refused
    narrow = B.MXGemmConfig(4, 1, 128)
    assert L.mx_gemm_with_config(*dict(args, m=0).values(), ctypes.byref(narrow), NULL) == B.MX_OK
    assert L.mx_gemm_with_config(*dict(args, m=0, epi=1).values(), ctypes.byref(narrow), NULL) == B.MX_OK
    assert L.mx_gemm_with_config(*dict(args, m=0, out_kind=2, out_scales=FAKE).values(), ctypes.byref(narrow),
                                 NULL) == B.MX_OK
    assert L.mx_gemm_with_config(*dict(args, epi=2, n=128, m=0).values(), ctypes.byref(narrow), NULL) == B.MX_OK
    assert L.mx_gemm_with_config(*dict(args, a_fmt=0, w_fmt=0).values(), ctypes.byref(narrow),
                                 NULL) == B.MX_ERR_UNSUPPORTED
    # eight waves: 256-feature tiles of every pair and epilogue, not with 128-feature tiles
    eight = B.MXGemmConfig(4, 1, 256, 8)
    assert L.mx_gemm_with_config(*dict(args, m=0).values(), ctypes.byref(eight), NULL) == B.MX_OK
    assert L.mx_gemm_with_config(*dict(args, m=0, a_fmt=0, w_fmt=0).values(), ctypes.byref(eight),
                                 NULL) == B.MX_OK
    assert L.mx_gemm_with_config(*dict(args, epi=2, n=128, m=0).values(), ctypes.byref(eight),
                                 NULL) == B.MX_OK
    assert L.mx_gemm_with_config(*dict(args, epi=2, n=192).values(), ctypes.byref(eight),
                                 NULL) == B.MX_ERR_UNSUPPORTED  # gate/up runs of 128 rows
    narrow8 = B.MXGemmConfig(4, 1, 128, 8)
    assert L.mx_gemm_with_config(*dict(args, m=0).values(), ctypes.byref(narrow8), NULL) == B.MX_ERR_UNSUPPORTED


def sk(**kw):
    a = dict(a_src=NULL, a_src_type=0, lda=0, a_codes=FAKE, a_scales=FAKE, a_fmt=2, w_codes=FAKE, w_scales=FAKE,
             w_fmt=3, m=16, n=64, k=4096, splits=8, out_kind=1, out=FAKE, ldo=64, ws=FAKE, ws_bytes=1 << 30,
             stream=NULL)
    a.update(kw)
    return mx.lib().mx_gemm_splitk(*a.values())


@host_only
def test_splitk_validation(L):
    assert sk(m=17) == B.MX_ERR_SHAPE
    assert sk(splits=0) == B.MX_ERR_SHAPE
    assert sk(splits=3) == B.MX_ERR_UNSUPPORTED
    assert sk(splits=64) == B.MX_ERR_UNSUPPORTED  # 64-element chunks (not whole 128-element stages)
    assert sk(splits=32) == B.MX_ERR_UNSUPPORTED  # at most 16 chunks
    assert sk(out_kind=2) == B.MX_ERR_FORMAT
    # activations quantized inside the call need a workspace
    src = dict(a_src=FAKE, lda=4096, a_codes=NULL, a_scales=NULL)
    assert sk(ws_bytes=10, **src) == B.MX_ERR_WORKSPACE
    assert sk(ws=NULL, **src) == B.MX_ERR_WORKSPACE
    assert sk(ws=FAKE + 16, **src) == B.MX_ERR_ALIGN
    assert sk(a_fmt=3) == B.MX_ERR_UNSUPPORTED
    assert sk(a_fmt=0, w_fmt=0) == B.MX_ERR_UNSUPPORTED  # 6-bit types only
    assert sk(m=0) == B.MX_OK


def sk_noalloc(**kw):
    a = dict(a_src=FAKE, a_src_type=0, lda=1 << 17, a_codes=NULL, a_scales=NULL, a_fmt=2, w_codes=FAKE,
             w_scales=FAKE, w_fmt=3, m=16, n=64, k=4096, splits=8, out_kind=1, out=FAKE, ldo=64, stream=NULL)
    a.update(kw)
    return mx.lib().mx_gemm_splitk_noalloc(*a.values())


@host_only
def test_splitk_noalloc_validation(L):
    """The allocation-free split-K entry point validates like mx_gemm_splitk
    (on the host, before any HIP call) and refuses a K beyond its static
    scratch with its own status."""
    assert B.MX_NOALLOC_MAX_K == 65536
    assert sk_noalloc(k=B.MX_NOALLOC_MAX_K + 1024) == B.MX_ERR_SCRATCH
    assert sk_noalloc(k=1 << 20, lda=1 << 20, splits=16) == B.MX_ERR_SCRATCH
    assert "scratch" in mx.mx_status_string(B.MX_ERR_SCRATCH)
    assert sk_noalloc(m=17) == B.MX_ERR_SHAPE
    assert sk_noalloc(splits=3) == B.MX_ERR_UNSUPPORTED
    assert sk_noalloc(out_kind=2) == B.MX_ERR_FORMAT
    assert sk_noalloc(out=NULL) == B.MX_ERR_NULL
    assert sk_noalloc(a_src=FAKE + 8) == B.MX_ERR_ALIGN
    assert sk_noalloc(a_fmt=3) == B.MX_ERR_UNSUPPORTED
    assert sk_noalloc(m=0) == B.MX_OK  # nothing to do: no HIP call


@host_only
def test_size_limits_rejected_before_launch(L):
    """Requests past the launch limits (a kernel of 2^32 lanes or more, one
    GEMM operand stage of 4 GiB or more, a tiled matrix of 2^40 code bytes or
    more) return MX_ERR_UNSUPPORTED on the host, before anything is launched;
    a dimension above 2^30 is MX_ERR_SHAPE."""
    s = NULL
    # rows layout: one lane per 32-element block; 2^27 rows x 32 blocks = 2^32 lanes
    assert q(FAKE, 0, 1 << 27, 1024, 1024, 2, 0, FAKE, FAKE, s) == B.MX_ERR_UNSUPPORTED
    # tiled layout: 2^23 stages x 2^25 groups of 3072 bytes
    assert q(FAKE, 0, 1 << 30, 1 << 30, 1 << 30, 2, 1, FAKE, FAKE, s) == B.MX_ERR_UNSUPPORTED
    assert q(FAKE, 0, (1 << 30) + 1, 64, 64, 2, 1, FAKE, FAKE, s) == B.MX_ERR_SHAPE
    # producer: bf16 rows of up to 3072 take 2 x 512 lanes per 32-row group
    assert rq(rows=1 << 27, d=32, ld=32) == B.MX_ERR_UNSUPPORTED
    # fp32 (the two-pass kernel): 256 lanes per group
    assert rq(rows=1 << 30, d=32, ld=32, src_type=1) == B.MX_ERR_UNSUPPORTED
    # GEMM: 2^14 x 2^14 tiles of 256 lanes; a stage of 2^21 row groups x 3072 bytes
    assert g(m=1 << 22, n=1 << 22, ldo=1 << 22) == B.MX_ERR_UNSUPPORTED
    assert g(m=1 << 26, n=64) == B.MX_ERR_UNSUPPORTED
    assert g(m=64, n=1 << 26, ldo=1 << 26) == B.MX_ERR_UNSUPPORTED
    assert g(m=1 << 25, n=1 << 25, ldo=1 << 25) == B.MX_ERR_SHAPE  # 2^34 tiles
    # split-K: one workgroup of 256 lanes per 64 weight rows
    assert sk(n=1 << 30, k=128, splits=1, ldo=1 << 30) == B.MX_ERR_UNSUPPORTED
    # leading dimensions are dimensions too: above 2^30 elements is MX_ERR_SHAPE
    big = (1 << 30) + 64
    assert q(FAKE, 0, 4, 64, big, 2, 1, FAKE, FAKE, s) == B.MX_ERR_SHAPE
    assert q(FAKE, 1, 4, 64, big, 2, 0, FAKE, FAKE, s) == B.MX_ERR_SHAPE
    assert rq(ld=big) == B.MX_ERR_SHAPE
    assert g(a_src=FAKE, lda=big, a_codes=NULL, a_scales=NULL) == B.MX_ERR_SHAPE
    assert g(ldo=big) == B.MX_ERR_SHAPE
    assert g(out_kind=0, ldo=big) == B.MX_ERR_SHAPE
    assert sk(ldo=big) == B.MX_ERR_SHAPE
    assert sk(a_src=FAKE, lda=big, a_codes=NULL, a_scales=NULL) == B.MX_ERR_SHAPE
    assert sk_noalloc(lda=big) == B.MX_ERR_SHAPE


def test_abi_from_plain_c(L, tmp_path):
    """tests/abi_from_c.c: the header compiles as C99 with gcc, the program
    links against libmxgemm.so, and the calls that need no device (version,
    status strings, sizes, configurations, argument errors) answer as the
    header says."""
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "abi_from_c"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "abi_from_c.c"), "-L", os.path.dirname(B.LIB_PATH),
           "-lmxgemm", f"-Wl,-rpath,{os.path.dirname(B.LIB_PATH)}", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.count("ok  ") == 16, run.stdout


def test_packed_bytes(L):
    assert mx.mx_packed_bytes(300, 416, "rows", 0) == 300 * 416 * 3 // 4
    assert mx.mx_packed_bytes(300, 416, "rows", 1) == 300 * 13
    # tiled: ceil(416/128) = 4 stages x ceil(300/32) = 10 groups
    assert mx.mx_packed_bytes(300, 416, "tiled", 0) == 4 * 10 * 3072
    assert mx.mx_packed_bytes(300, 416, "tiled", 1) == 4 * 10 * 128
    assert mx.mx_packed_bytes(300, 100, "tiled", 0) == 0  # invalid K
    assert mx.lib().mx_packed_bytes(10, 64, 2, 5, 0) == 0  # bad layout
    assert mx.lib().mx_packed_bytes(10, 64, 2, 1, 2) == 0  # bad selector
    assert mx.lib().mx_packed_bytes(10, 64, 7, 1, 0) == 0  # bad format
    # 4- and 8-bit element types: 16 / 32 code bytes per block, chunks of 2048 / 4096
    assert mx.mx_packed_bytes(300, 416, "rows", 0, "e2m1") == 300 * 416 // 2
    assert mx.mx_packed_bytes(300, 416, "rows", 0, "e4m3") == 300 * 416
    assert mx.mx_packed_bytes(300, 416, "tiled", 0, "e2m1") == 4 * 10 * 2048
    assert mx.mx_packed_bytes(300, 416, "tiled", 0, "e5m2") == 4 * 10 * 4096
    assert mx.mx_packed_bytes(300, 416, "tiled", 1, "e4m3") == 4 * 10 * 128


def test_workspace_sizes(L):
    assert mx.mx_gemm_workspace_size(64, 64, 128, False, 0) == 0
    assert mx.mx_gemm_workspace_size(64, 64, 100, True, 0) == 0  # invalid K
    assert mx.mx_gemm_workspace_size(17, 64, 128, True, 4) == 0  # splitk needs m <= 16
    assert mx.mx_gemm_workspace_size(16, 64, 128, True, 17) == 0  # at most 16 chunks
    # split-K keeps its partial sums on chip: the workspace only holds the
    # activations quantized in the call (128 stages x one 32-row group)
    sz = mx.mx_gemm_workspace_size(16, 13312, 16384, True, 16)
    assert sz == mx.mx_gemm_workspace_size(16, 13312, 16384, True, 0) >= 128 * (4096 + 128)
    assert mx.mx_gemm_workspace_size(16, 13312, 16384, False, 16) == 0


def test_binding_refuses_cpu_tensors(L):
    import torch
    with pytest.raises(ValueError):
        mx.mx_quantize(torch.zeros(4, 64, dtype=torch.bfloat16))


def test_quantize_and_producer_bindings_check_out_before_launch(L):
    """A caller-supplied out of the quantizer and of the producer must match
    the call's element format (codes of another width would be written past
    its buffers), shape and layout, and live on the GPU like the inputs;
    the producer's vectors must be contiguous fp32 of d features."""
    import torch
    x = torch.zeros(32, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="element format"):
        mx.mx_quantize(x, "e4m3", "tiled", out=_cpu_mx(32, 128, "e2m1"))   # 8-bit codes into a 4-bit buffer
    with pytest.raises(ValueError, match="shape"):
        mx.mx_quantize(x, "e2m3", "tiled", out=_cpu_mx(32, 96))
    with pytest.raises(ValueError, match="GPU"):
        mx.mx_quantize(x, "e2m3", "tiled", out=_cpu_mx(32, 128))
    with pytest.raises(ValueError, match="MX matrix"):
        mx.mx_rmsnorm_quantize(x, fmt="e3m2", out=_cpu_mx(32, 128, "e2m3"))
    with pytest.raises(ValueError, match="fp32"):
        mx.mx_rmsnorm_quantize(x, gamma=torch.ones(128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="features"):
        mx.mx_rmsnorm_quantize(x, gamma=torch.ones(64, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        mx.mx_rmsnorm_quantize(x, gamma=torch.ones(128, dtype=torch.float32), out=_cpu_mx(32, 128))
    with pytest.raises(ValueError, match="gamma"):
        mx.mx_rmsnorm_quantize(x, gamma=torch.ones(2, 128, dtype=torch.float32))
    # the kernel reads conditioning row r // rows_per_cond for every row r: 96
    # rows at 32 rows per conditioning need 3 rows of shift and of scale
    x96 = torch.zeros(96, 128, dtype=torch.bfloat16)
    two = torch.zeros(2, 128, dtype=torch.float32)
    with pytest.raises(ValueError, match="shift must hold"):
        mx.mx_rmsnorm_quantize(x96, shift=two, rows_per_cond=32)
    with pytest.raises(ValueError, match="scale must hold"):
        mx.mx_rmsnorm_quantize(x96, scale=torch.zeros(128, dtype=torch.float32), rows_per_cond=64)
    with pytest.raises(ValueError, match="GPU"):  # 2 rows at 64 rows per conditioning: sizes pass
        mx.mx_rmsnorm_quantize(x96, shift=two, scale=two, rows_per_cond=64)


def _cpu_mx(rows, k, fmt="e2m3"):
    import torch
    return B.MXTensor(torch.zeros(mx.mx_packed_bytes(rows, k, "tiled", 0, fmt), dtype=torch.uint8),
                      torch.zeros(mx.mx_packed_bytes(rows, k, "tiled", 1, fmt), dtype=torch.uint8), fmt, rows, k)


@pytest.mark.parametrize("fn", ["gemm", "splitk"])
def test_binding_checks_out_workspace_and_k_before_launch(L, fn):
    """Every malformed argument of the Python wrappers is refused with a
    ValueError naming it, before any pointer reaches the library: a wrong
    out dtype, rank, shape or stride (which would be written out of bounds),
    a K mismatch between MX operands (read past A), a non-uint8 workspace
    (its numel would not be its byte count), and CPU buffers anywhere."""
    import torch
    m, n, k = 16, 64, 256
    w = _cpu_mx(n, k)
    a = _cpu_mx(m, k)
    call = (lambda **kw: mx.mx_gemm(a, w, out_kind="f32", **kw)) if fn == "gemm" else \
        (lambda **kw: mx.mx_gemm_splitk(a, w, 2, out_kind="f32", **kw))
    bad_outs = [torch.zeros(m, n, dtype=torch.bfloat16),          # bf16 buffer for fp32 output
                torch.zeros(m, n - 1, dtype=torch.float32),       # too narrow
                torch.zeros(m - 1, n, dtype=torch.float32),       # too few rows
                torch.zeros(n, m, dtype=torch.float32).t(),       # column stride
                torch.zeros(m * n, dtype=torch.float32)]          # 1-D
    for o in bad_outs:
        with pytest.raises(ValueError, match="out must be"):
            call(out=o)
    with pytest.raises(ValueError, match="workspace"):
        call(workspace=torch.zeros(64, dtype=torch.float32))
    # right shapes, CPU buffers: refused by the device check
    with pytest.raises(ValueError, match="GPU"):
        call(out=torch.zeros(m, n, dtype=torch.float32))
    # K mismatch between the MX activations and the weights
    a_short = _cpu_mx(m, k - 128)
    with pytest.raises(ValueError, match="disagree on K"):
        if fn == "gemm":
            mx.mx_gemm(a_short, w, out_kind="f32")
        else:
            mx.mx_gemm_splitk(a_short, w, 2, out_kind="f32")
    if fn == "splitk":
        with pytest.raises(ValueError, match="fp32 or bf16"):
            mx.mx_gemm_splitk(a, w, 2, out_kind="mx")
    else:
        # MX output: an out of the wrong kind or element format
        with pytest.raises(ValueError):
            mx.mx_gemm(a, w, out_kind="mx", out=torch.zeros(m, n, dtype=torch.float32))
        with pytest.raises(ValueError, match="MX matrix"):
            mx.mx_gemm(a, w, out_kind="mx", out_fmt="e2m3", out=_cpu_mx(m, n, "e3m2"))
        with pytest.raises(ValueError, match="MX matrix"):
            mx.mx_gemm(a, w, out_kind="mx", out=_cpu_mx(m, n - 32))


def test_launch_log(L):
    """MXGEMM_LOG=1 makes every computing call write one line to stderr with
    its sizes and status (checked in a child process, on calls that fail
    validation, so nothing is launched); without it the library is silent."""
    import subprocess
    import sys
    code = (
        "import microscaled_precision_gemm_amd as mx, ctypes\n"
        "L = mx.lib()\n"
        "print(L.mx_quantize(None, 0, 4, 48, 48, 2, 1, None, None, None))\n"       # k % 32 != 0
        "print(L.mx_gemm(None, 0, 0, None, None, 3, None, None, 3, 4, 64, 128, 0, 1, None, 64, None, 2, None, 0,"
        " None))\n"                                                                   # E3M2 x E3M2
        "print(L.mx_gemm_splitk(None, 0, 0, None, None, 2, None, None, 3, 17, 64, 0, 1, 1, None, 64, None, 0,"
        " None))\n")                                                                  # m > 16
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, MXGEMM_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == [str(B.MX_ERR_SHAPE), str(B.MX_ERR_UNSUPPORTED), str(B.MX_ERR_SHAPE)]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("mxgemm: ")]
    assert len(lines) == 3, r.stderr
    assert lines[0].startswith("mxgemm: mx_quantize rows=4 k=48 ") and lines[0].endswith(f"-> {B.MX_ERR_SHAPE} "
                                                                                          f"({mx.mx_status_string(B.MX_ERR_SHAPE)})")
    assert lines[1].startswith("mxgemm: mx_gemm m=4 n=64 k=128 a=mx fmt=3 w_fmt=3") and "by shape rule" in lines[1]
    assert lines[2].startswith("mxgemm: mx_gemm_splitk m=17 ")
    env.pop("MXGEMM_LOG")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "mxgemm:" not in r.stderr
