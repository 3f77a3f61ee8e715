// MX GEMM variants: FP8 weights x FP8 activations, E4M3 and E5M2 in every pairing.
#include "gemm_kernel.h"

namespace mxg {
template hipError_t launch_gemm_formats<kFmtE4M3, kFmtE4M3>(const GemmArgs&, int, int, int, hipStream_t);
template hipError_t launch_gemm_formats<kFmtE5M2, kFmtE5M2>(const GemmArgs&, int, int, int, hipStream_t);
template hipError_t launch_gemm_formats<kFmtE4M3, kFmtE5M2>(const GemmArgs&, int, int, int, hipStream_t);
template hipError_t launch_gemm_formats<kFmtE5M2, kFmtE4M3>(const GemmArgs&, int, int, int, hipStream_t);
}  // namespace mxg
