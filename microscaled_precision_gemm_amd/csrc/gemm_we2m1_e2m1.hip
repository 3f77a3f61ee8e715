// MX GEMM variant: FP4 (E2M1) weights x FP4 (E2M1) activations.
#include "gemm_kernel.h"

namespace mxg {
template hipError_t launch_gemm_formats<kFmtE2M1, kFmtE2M1>(const GemmArgs&, int, int, int, hipStream_t);
}  // namespace mxg
