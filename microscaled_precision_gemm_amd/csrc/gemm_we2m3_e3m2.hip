// MX GEMM kernels for weights e2m3 x activations e3m2 (see gemm_kernel.h).
#include "gemm_kernel.h"

namespace mxg {
template hipError_t launch_gemm_formats<kFmtE2M3, kFmtE3M2>(const GemmArgs&, int, int, int, hipStream_t);
}  // namespace mxg
