"""MXFP6 block-scaled GEMM for AMD Instinct MI355X (gfx950).

The compute lives in ``libmxgemm.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/mxgemm.h``); this package is its ctypes binding.
"""

from .binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    MXError,
    MXGemmConfig,
    MXTensor,
    lib,
    mx_gemm,
    mx_gemm_default_config,
    mx_gemm_select_config,
    mx_gemm_splitk,
    mx_gemm_workspace_size,
    mx_packed_bytes,
    mx_quantize,
    mx_rmsnorm_quantize,
    mx_status_string,
    mx_version,
)
