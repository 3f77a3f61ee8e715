"""ctypes binding of libmxgemm.so, with the same names as the C ABI.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs and workspaces are allocated with torch (device memory is
torch's job here), and every computation runs in the library's HIP kernels on
torch's current stream.  There is no CPU fallback: without the built library
every call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxgemm.so")

MX_OK = 0
MX_ERR_NULL = -1
MX_ERR_SHAPE = -2
MX_ERR_FORMAT = -3
MX_ERR_ALIGN = -4
MX_ERR_WORKSPACE = -5
MX_ERR_UNSUPPORTED = -6
MX_ERR_HIP = -7
MX_ERR_SCRATCH = -8
MX_NOALLOC_MAX_K = 65536

MX_FMT_E4M3 = 0
MX_FMT_E5M2 = 1
MX_FMT_E2M3 = 2
MX_FMT_E3M2 = 3
MX_FMT_E2M1 = 4
MX_SRC_BF16 = 0
MX_SRC_F32 = 1
MX_OUT_F32 = 0
MX_OUT_BF16 = 1
MX_OUT_MX = 2
MX_EPI_NONE = 0
MX_EPI_GELU_TANH = 1
MX_EPI_SWIGLU = 2
MX_LAYOUT_ROWS = 0
MX_LAYOUT_TILED = 1

FMT_CODES = {"e2m3": MX_FMT_E2M3, "e3m2": MX_FMT_E3M2, "e2m1": MX_FMT_E2M1, "e4m3": MX_FMT_E4M3,
             "e5m2": MX_FMT_E5M2}
FMT_BITS = {"e2m3": 6, "e3m2": 6, "e2m1": 4, "e4m3": 8, "e5m2": 8}
OUT_KINDS = {"f32": MX_OUT_F32, "bf16": MX_OUT_BF16, "mx": MX_OUT_MX}
EPILOGUES = {"none": MX_EPI_NONE, "gelu_tanh": MX_EPI_GELU_TANH, "swiglu": MX_EPI_SWIGLU}
LAYOUTS = {"rows": MX_LAYOUT_ROWS, "tiled": MX_LAYOUT_TILED}

EXPORTED = ("mx_quantize", "mx_rmsnorm_quantize", "mx_packed_bytes", "mx_gemm", "mx_gemm_default_config",
            "mx_gemm_select_config", "mx_gemm_with_config", "mx_gemm_splitk", "mx_gemm_splitk_noalloc", "mx_gemm_workspace_size",
            "mx_status_string", "mx_version")


class MXGemmConfig(ctypes.Structure):
    """mx_gemm_config: the tile order, tile width and waves per workgroup of
    mx_gemm (speed only, never the result).  Built from (group_m, xcd_remap[,
    tile_n[, waves]]); tile_n defaults to 256, waves to 4."""

    _fields_ = [("group_m", ctypes.c_int32), ("xcd_remap", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("waves", ctypes.c_int32)]

    def __init__(self, group_m: int = 4, xcd_remap: int = 1, tile_n: int = 256, waves: int = 4):
        super().__init__(group_m, xcd_remap, tile_n, waves)

    def key(self) -> tuple[int, int, int, int]:
        return (int(self.group_m), int(self.xcd_remap), int(self.tile_n), int(self.waves))


class MXError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {mx_status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmxgemm.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built: run `python -m microscaled_precision_gemm_amd.build` "
            "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    c_i32, c_i64, c_p, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    L.mx_quantize.argtypes = [c_p, c_i32, c_i64, c_i64, c_i64, c_i32, c_i32, c_p, c_p, c_p]
    L.mx_quantize.restype = ctypes.c_int
    L.mx_rmsnorm_quantize.argtypes = [c_p, c_i32, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_i64, ctypes.c_float, c_i32,
                                      c_p, c_p, c_p]
    L.mx_rmsnorm_quantize.restype = ctypes.c_int
    L.mx_packed_bytes.argtypes = [c_i64, c_i64, c_i32, c_i32, c_i32]
    L.mx_packed_bytes.restype = c_sz
    L.mx_gemm.argtypes = [c_p, c_i32, c_i64, c_p, c_p, c_i32, c_p, c_p, c_i32, c_i64, c_i64, c_i64, c_i32, c_i32,
                          c_p, c_i64, c_p, c_i32, c_p, c_sz, c_p]
    L.mx_gemm.restype = ctypes.c_int
    L.mx_gemm_with_config.argtypes = L.mx_gemm.argtypes[:-1] + [ctypes.POINTER(MXGemmConfig), c_p]
    L.mx_gemm_with_config.restype = ctypes.c_int
    L.mx_gemm_default_config.argtypes = [ctypes.POINTER(MXGemmConfig)]
    L.mx_gemm_default_config.restype = None
    L.mx_gemm_select_config.argtypes = [c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(MXGemmConfig)]
    L.mx_gemm_select_config.restype = None
    L.mx_gemm_splitk.argtypes = [c_p, c_i32, c_i64, c_p, c_p, c_i32, c_p, c_p, c_i32, c_i64, c_i64, c_i64, c_i32,
                                 c_i32, c_p, c_i64, c_p, c_sz, c_p]
    L.mx_gemm_splitk.restype = ctypes.c_int
    L.mx_gemm_splitk_noalloc.argtypes = L.mx_gemm_splitk.argtypes[:16] + [c_p]
    L.mx_gemm_splitk_noalloc.restype = ctypes.c_int
    L.mx_gemm_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_i32, c_i32]
    L.mx_gemm_workspace_size.restype = c_sz
    L.mx_status_string.argtypes = [ctypes.c_int]
    L.mx_status_string.restype = ctypes.c_char_p
    L.mx_version.argtypes = []
    L.mx_version.restype = ctypes.c_int
    _lib = L
    return L


def mx_status_string(status: int) -> str:
    return lib().mx_status_string(int(status)).decode()


def mx_version() -> int:
    return int(lib().mx_version())


def mx_gemm_workspace_size(m: int, n: int, k: int, a_is_src: bool, splits: int = 0) -> int:
    return int(lib().mx_gemm_workspace_size(m, n, k, int(bool(a_is_src)), splits))


def mx_packed_bytes(rows: int, k: int, layout: str = "tiled", which: int = 0, fmt: str = "e2m3") -> int:
    """Bytes of the codes (which=0) or scales (which=1) buffer of a [rows, k] MX matrix."""
    return int(lib().mx_packed_bytes(rows, k, _fmt(fmt), LAYOUTS[layout], which))


@dataclass
class MXTensor:
    """Packed MX matrix of logical shape [rows, k].

    layout "rows": codes [rows, b*k/8] (b = 6, 4 or 8 bits per element) and
    scales [rows, k/32] uint8 tensors.
    layout "tiled": codes and scales are flat uint8 tensors in the tiled GEMM
    layout (128-element stages x 32-row groups, see include/mxgemm.h).
    """

    codes: torch.Tensor
    scales: torch.Tensor
    fmt: str
    rows: int
    k: int
    layout: str = "tiled"

    @staticmethod
    def empty(rows: int, k: int, fmt: str = "e2m3", layout: str = "tiled", device=None) -> "MXTensor":
        if layout == "rows":
            codes = torch.empty((rows, FMT_BITS[fmt] * k // 8), dtype=torch.uint8, device=device)
            scales = torch.empty((rows, k // 32), dtype=torch.uint8, device=device)
        else:
            codes = torch.empty(mx_packed_bytes(rows, k, layout, 0, fmt), dtype=torch.uint8, device=device)
            scales = torch.empty(mx_packed_bytes(rows, k, layout, 1, fmt), dtype=torch.uint8, device=device)
        return MXTensor(codes, scales, fmt, rows, k, layout)


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else None)


def _check(status: int, where: str) -> None:
    if status != MX_OK:
        raise MXError(status, where)


def _fmt(fmt: str) -> int:
    try:
        return FMT_CODES[fmt]
    except KeyError:
        raise ValueError(f"unknown MX format {fmt!r}") from None


def _src_type(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MX_SRC_BF16
    if t.dtype == torch.float32:
        return MX_SRC_F32
    raise TypeError(f"unsupported source dtype {t.dtype}; expected bfloat16 or float32")


def _require_cuda(*ts: torch.Tensor | None) -> torch.device:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU (no CPU fallback)")
        dev = t.device if dev is None else dev
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _mx_parts(x: MXTensor | None) -> tuple[torch.Tensor | None, torch.Tensor | None]:
    return (x.codes, x.scales) if x is not None else (None, None)


def _check_workspace(workspace: torch.Tensor | None) -> None:
    """A caller-supplied workspace is a contiguous uint8 buffer: its numel()
    is the byte count handed to the library."""
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor")


def _check_plain_out(out: torch.Tensor, dtype: torch.dtype, m: int, n: int) -> None:
    if out.dtype != dtype or out.dim() != 2 or out.stride(1) != 1 or tuple(out.shape) != (m, n):
        raise ValueError(f"out must be a [{m}, {n}] {dtype} tensor with unit stride along its rows")


def _check_mx(x: MXTensor, name: str, layout: str | None = None) -> None:
    if layout is not None and x.layout != layout:
        raise ValueError(f"{name}: expected the {layout!r} layout, got {x.layout!r}")
    if x.codes.dtype != torch.uint8 or x.scales.dtype != torch.uint8:
        raise TypeError(f"{name}: codes and scales must be uint8")
    if not (x.codes.is_contiguous() and x.scales.is_contiguous()):
        raise ValueError(f"{name}: codes and scales must be contiguous")
    if x.layout == "rows":
        ok = (tuple(x.codes.shape) == (x.rows, FMT_BITS[x.fmt] * x.k // 8)
              and tuple(x.scales.shape) == (x.rows, x.k // 32))
    else:
        ok = (x.codes.numel() == mx_packed_bytes(x.rows, x.k, x.layout, 0, x.fmt)
              and x.scales.numel() == mx_packed_bytes(x.rows, x.k, x.layout, 1, x.fmt))
    if not ok:
        raise ValueError(f"{name}: buffer sizes do not match a [{x.rows}, {x.k}] {x.layout} MX matrix")


def mx_quantize(src: torch.Tensor, fmt: str = "e2m3", layout: str = "tiled", out: MXTensor | None = None) -> MXTensor:
    """MX-quantize a 2-D bf16/fp32 GPU tensor along its rows (blocks of 32)."""
    if src.dim() != 2 or src.stride(1) != 1:
        raise ValueError("src must be 2-D with unit stride along K")
    rows, k = src.shape
    if out is not None:
        # the kernel writes `fmt` codes: an out sized for another element width would overflow
        if out.rows != rows or out.k != k or out.layout != layout or out.fmt != fmt:
            raise ValueError("out does not match the source shape / layout / element format")
        _check_mx(out, "out")
    dev = _require_cuda(src, *_mx_parts(out))
    if out is None:
        out = MXTensor.empty(rows, k, fmt, layout, dev)
    st = lib().mx_quantize(_ptr(src), _src_type(src), rows, k, src.stride(0), _fmt(fmt), LAYOUTS[layout],
                           _ptr(out.codes), _ptr(out.scales), _stream(dev))
    _check(st, "mx_quantize")
    return out


def mx_rmsnorm_quantize(x: torch.Tensor, gamma: torch.Tensor | None = None, shift: torch.Tensor | None = None,
                        scale: torch.Tensor | None = None, rows_per_cond: int = 0, eps: float = 1e-6,
                        fmt: str = "e2m3", out: MXTensor | None = None) -> MXTensor:
    """RMSNorm + modulation + MX quantization of x [rows, d] into the tiled
    layout (the GEMM operand).  gamma: fp32 [d]; shift / scale: fp32
    [n_cond, d] with rows_per_cond rows per conditioning row (a multiple of 32)."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [rows, d] with unit stride along d")
    rows, d = x.shape
    for name, v in (("gamma", gamma), ("shift", shift), ("scale", scale)):
        if v is not None:
            if v.dtype != torch.float32 or not v.is_contiguous():
                raise ValueError(f"{name} must be a contiguous fp32 tensor")
            if v.shape[-1] != d:
                raise ValueError(f"{name} must have d = {d} features")
    if gamma is not None and gamma.numel() != d:
        raise ValueError(f"gamma must be [{d}]")
    if rows_per_cond > 0 and rows > 0:
        # the kernel reads conditioning row r // rows_per_cond for every row r
        n_cond = -(-rows // rows_per_cond)
        for name, v in (("shift", shift), ("scale", scale)):
            if v is not None and v.numel() < n_cond * d:
                raise ValueError(f"{name} must hold ceil(rows / rows_per_cond) = {n_cond} rows of {d} features")
    if out is not None:
        if out.rows != rows or out.k != d or out.layout != "tiled" or out.fmt != fmt:
            raise ValueError(f"out must be a tiled [rows, d] {fmt} MX matrix")
        _check_mx(out, "out")
    dev = _require_cuda(x, gamma, shift, scale, *_mx_parts(out))
    if out is None:
        out = MXTensor.empty(rows, d, fmt, "tiled", dev)
    st = lib().mx_rmsnorm_quantize(_ptr(x), _src_type(x), rows, d, x.stride(0), _ptr(gamma), _ptr(shift), _ptr(scale),
                                   rows_per_cond, float(eps), _fmt(fmt), _ptr(out.codes), _ptr(out.scales),
                                   _stream(dev))
    _check(st, "mx_rmsnorm_quantize")
    return out


def mx_gemm_default_config() -> MXGemmConfig:
    """The generic launch configuration (every format pair and epilogue)."""
    c = MXGemmConfig()
    lib().mx_gemm_default_config(ctypes.byref(c))
    return c


def mx_gemm_select_config(m: int, n: int, k: int, a_fmt: str = "e2m3", w_fmt: str = "e2m3", epilogue: str = "none",
                          out_kind: str = "bf16") -> MXGemmConfig:
    """The configuration mx_gemm uses for this call shape when given none
    (the library's shape rule)."""
    c = MXGemmConfig()
    lib().mx_gemm_select_config(m, n, k, _fmt(a_fmt), _fmt(w_fmt), EPILOGUES[epilogue], OUT_KINDS[out_kind],
                                ctypes.byref(c))
    return c


def mx_gemm(a: torch.Tensor | MXTensor, w: MXTensor, out_kind: str = "bf16", epilogue: str = "none",
            out_fmt: str = "e2m3", a_fmt: str = "e2m3", out: torch.Tensor | MXTensor | None = None,
            workspace: torch.Tensor | None = None, config: MXGemmConfig | tuple[int, ...] | None = None):
    """C = A W^T.  ``a`` is a bf16/fp32 tensor (quantized to ``a_fmt`` inside the
    call) or an MXTensor.  Returns a [m, n_out] tensor, or an MXTensor for
    out_kind="mx"; n_out = n, or n / 2 for epilogue="swiglu" (``w`` then holds
    stacked gate/up rows, see include/mxgemm.h).  ``config``: the tile order
    and shape (an MXGemmConfig or (group_m, xcd_remap[, tile_n[, waves]]));
    None = the library's shape rule (mx_gemm_select_config)."""
    _check_mx(w, "w", "tiled")
    n, k = w.rows, w.k
    n_out = n // 2 if epilogue == "swiglu" else n
    if isinstance(a, MXTensor):
        _check_mx(a, "a", "tiled")
        a_src, a_codes, a_scales, af, lda, m = None, a.codes, a.scales, _fmt(a.fmt), 0, a.rows
        if a.k != k:
            raise ValueError("A and W disagree on K")
        src_type = MX_SRC_BF16
    else:
        if a.dim() != 2 or a.stride(1) != 1 or a.shape[1] != k:
            raise ValueError("a must be [m, k] with unit stride along K")
        a_src, a_codes, a_scales, af, lda, m = a, None, None, _fmt(a_fmt), a.stride(0), a.shape[0]
        src_type = _src_type(a)
    kind = OUT_KINDS[out_kind]
    if kind == MX_OUT_MX and out is not None and not isinstance(out, MXTensor):
        raise ValueError("out_kind='mx' needs an MXTensor out")
    if kind != MX_OUT_MX and isinstance(out, MXTensor):
        raise ValueError(f"out_kind={out_kind!r} needs a tensor out")
    # every shape / dtype check first, then one device check over every buffer
    _check_workspace(workspace)
    dtype = torch.float32 if kind == MX_OUT_F32 else torch.bfloat16
    if out is not None:
        if kind == MX_OUT_MX:
            _check_mx(out, "out", "tiled")
            if out.rows != m or out.k != n_out or out.fmt != out_fmt:
                raise ValueError(f"out must be an [m, n_out] {out_fmt} MX matrix")
        else:
            _check_plain_out(out, dtype, m, n_out)
    dev = _require_cuda(a_src, a_codes, a_scales, w.codes, w.scales, *_mx_parts(out if kind == MX_OUT_MX else None),
                        out if kind != MX_OUT_MX else None, workspace)
    if kind == MX_OUT_MX:
        if out is None:
            out = MXTensor.empty(m, n_out, out_fmt, "tiled", dev)
        out_data, out_scales, ldo = out.codes, out.scales, 0
    else:
        if out is None:
            out = torch.empty((m, n_out), dtype=dtype, device=dev)
        out_data, out_scales, ldo = out, None, out.stride(0)
    need = mx_gemm_workspace_size(m, n, k, a_src is not None, 0)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() if workspace is not None else 0
    args = (_ptr(a_src), src_type, lda, _ptr(a_codes), _ptr(a_scales), af, _ptr(w.codes), _ptr(w.scales),
            _fmt(w.fmt), m, n, k, EPILOGUES[epilogue], kind, _ptr(out_data), ldo, _ptr(out_scales), _fmt(out_fmt),
            _ptr(workspace), ws_bytes)
    if config is None:
        st = lib().mx_gemm(*args, _stream(dev))
    else:
        if not isinstance(config, MXGemmConfig):
            config = MXGemmConfig(*config)
        st = lib().mx_gemm_with_config(*args, ctypes.byref(config), _stream(dev))
    _check(st, "mx_gemm")
    return out


def mx_gemm_splitk(a: torch.Tensor | MXTensor, w: MXTensor, splits: int, out_kind: str = "bf16",
                   a_fmt: str = "e2m3", out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   noalloc: bool = False):
    """Skinny C = A W^T (m <= 16) with K split into ``splits`` chunks, fp32
    partials summed in a fixed order.  noalloc=True calls
    mx_gemm_splitk_noalloc instead (no workspace: the library's static
    scratch; ``out`` must then be given for the call itself to allocate
    nothing)."""
    _check_mx(w, "w", "tiled")
    n, k = w.rows, w.k
    if isinstance(a, MXTensor):
        _check_mx(a, "a", "tiled")
        a_src, a_codes, a_scales, af, lda, m = None, a.codes, a.scales, _fmt(a.fmt), 0, a.rows
        if a.k != k:
            raise ValueError("A and W disagree on K")
        src_type = MX_SRC_BF16
    else:
        if a.dim() != 2 or a.stride(1) != 1 or a.shape[1] != k:
            raise ValueError("a must be [m, k] with unit stride along K")
        a_src, a_codes, a_scales, af, lda, m = a, None, None, _fmt(a_fmt), a.stride(0), a.shape[0]
        src_type = _src_type(a)
    kind = OUT_KINDS[out_kind]
    if kind == MX_OUT_MX:
        raise ValueError("mx_gemm_splitk writes fp32 or bf16 output")
    _check_workspace(workspace)
    dtype = torch.float32 if kind == MX_OUT_F32 else torch.bfloat16
    if out is not None:
        _check_plain_out(out, dtype, m, n)
    dev = _require_cuda(a_src, a_codes, a_scales, w.codes, w.scales, out, workspace)
    if out is None:
        out = torch.empty((m, n), dtype=dtype, device=dev)
    if noalloc:
        if workspace is not None:
            raise ValueError("mx_gemm_splitk_noalloc takes no workspace")
        # the library's scratch is the current device's: make it the operands' device
        with torch.cuda.device(dev):
            st = lib().mx_gemm_splitk_noalloc(_ptr(a_src), src_type, lda, _ptr(a_codes), _ptr(a_scales), af,
                                              _ptr(w.codes), _ptr(w.scales), _fmt(w.fmt), m, n, k, splits, kind,
                                              _ptr(out), out.stride(0), _stream(dev))
        _check(st, "mx_gemm_splitk_noalloc")
        return out
    need = mx_gemm_workspace_size(m, n, k, a_src is not None, splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().mx_gemm_splitk(_ptr(a_src), src_type, lda, _ptr(a_codes), _ptr(a_scales), af, _ptr(w.codes),
                              _ptr(w.scales), _fmt(w.fmt), m, n, k, splits, kind, _ptr(out), out.stride(0),
                              _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(dev))
    _check(st, "mx_gemm_splitk")
    return out
