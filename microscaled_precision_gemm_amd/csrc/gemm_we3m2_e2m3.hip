// MX GEMM kernels for weights e3m2 x activations e2m3 (see gemm_kernel.h).
#include "gemm_kernel.h"

namespace mxg {
template hipError_t launch_gemm_formats<kFmtE3M2, kFmtE2M3>(const GemmArgs&, int, int, int, hipStream_t);
}  // namespace mxg
