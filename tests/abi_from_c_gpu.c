/* The hot path driven from plain C99 on the GPU, with no Python or torch in
 * the process: device memory from hipMalloc, the library's calls on a HIP
 * stream, results copied back and written out for the oracle to check.
 *
 *   abi_from_c_gpu IN OUT
 *
 * IN holds int32 m, n, k, then A (bf16 [m, k]) and W (bf16 [n, k]) as raw
 * little-endian bf16 bits.  The program quantizes W (E2M3, tiled), runs
 * mx_gemm with A quantized inside the call (fp32 out), runs mx_gemm_splitk on
 * A's first min(m, 16) rows with 4 splits (fp32 out), and writes the two fp32
 * results to OUT, one after the other.  Exit status 0 when every call
 * returned MX_OK. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "mxgemm.h"

#define CHECK_HIP(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
      return 2;                                                             \
    }                                                                       \
  } while (0)
#define CHECK_MX(x)                                                         \
  do {                                                                      \
    int s_ = (x);                                                           \
    if (s_ != MX_OK) {                                                      \
      fprintf(stderr, "%s: %s\n", #x, mx_status_string(s_));                \
      return 3;                                                             \
    }                                                                       \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 1;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 1;
  int32_t dims[3];
  if (fread(dims, sizeof dims, 1, f) != 1) return 1;
  const int64_t m = dims[0], n = dims[1], k = dims[2], ms = m < 16 ? m : 16;
  uint16_t* a_h = malloc((size_t)(m * k) * 2);
  uint16_t* w_h = malloc((size_t)(n * k) * 2);
  float* c_h = malloc((size_t)(m * n) * 4);
  float* s_h = malloc((size_t)(ms * n) * 4);
  if (!a_h || !w_h || !c_h || !s_h) return 1;
  if (fread(a_h, 2, (size_t)(m * k), f) != (size_t)(m * k) || fread(w_h, 2, (size_t)(n * k), f) != (size_t)(n * k))
    return 1;
  fclose(f);

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  void *a_d, *w_d, *wc_d, *c_d, *s_d, *wk_d, *wk2_d;
  uint8_t* wsc_d;
  const size_t wc_bytes = mx_packed_bytes(n, k, MX_FMT_E2M3, MX_LAYOUT_TILED, 0);
  const size_t wsc_bytes = mx_packed_bytes(n, k, MX_FMT_E2M3, MX_LAYOUT_TILED, 1);
  const size_t work = mx_gemm_workspace_size(m, n, k, 1, 0);
  const size_t work2 = mx_gemm_workspace_size(ms, n, k, 1, 4);
  CHECK_HIP(hipMalloc(&a_d, (size_t)(m * k) * 2));
  CHECK_HIP(hipMalloc(&w_d, (size_t)(n * k) * 2));
  CHECK_HIP(hipMalloc(&wc_d, wc_bytes));
  CHECK_HIP(hipMalloc((void**)&wsc_d, wsc_bytes));
  CHECK_HIP(hipMalloc(&c_d, (size_t)(m * n) * 4));
  CHECK_HIP(hipMalloc(&s_d, (size_t)(ms * n) * 4));
  CHECK_HIP(hipMalloc(&wk_d, work));
  CHECK_HIP(hipMalloc(&wk2_d, work2));
  CHECK_HIP(hipMemcpy(a_d, a_h, (size_t)(m * k) * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(w_d, w_h, (size_t)(n * k) * 2, hipMemcpyHostToDevice));

  CHECK_MX(mx_quantize(w_d, MX_SRC_BF16, n, k, k, MX_FMT_E2M3, MX_LAYOUT_TILED, wc_d, wsc_d, stream));
  CHECK_MX(mx_gemm(a_d, MX_SRC_BF16, k, NULL, NULL, MX_FMT_E2M3, wc_d, wsc_d, MX_FMT_E2M3, m, n, k, MX_EPI_NONE,
                   MX_OUT_F32, c_d, n, NULL, MX_FMT_E2M3, wk_d, work, stream));
  CHECK_MX(mx_gemm_splitk(a_d, MX_SRC_BF16, k, NULL, NULL, MX_FMT_E2M3, wc_d, wsc_d, MX_FMT_E2M3, ms, n, k, 4,
                          MX_OUT_F32, s_d, n, wk2_d, work2, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_HIP(hipMemcpy(c_h, c_d, (size_t)(m * n) * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(s_h, s_d, (size_t)(ms * n) * 4, hipMemcpyDeviceToHost));

  FILE* o = fopen(argv[2], "wb");
  if (!o) return 1;
  fwrite(c_h, 4, (size_t)(m * n), o);
  fwrite(s_h, 4, (size_t)(ms * n), o);
  fclose(o);
  hipFree(a_d);
  hipFree(w_d);
  hipFree(wc_d);
  hipFree(wsc_d);
  hipFree(c_d);
  hipFree(s_d);
  hipFree(wk_d);
  hipFree(wk2_d);
  hipStreamDestroy(stream);
  free(a_h);
  free(w_h);
  free(c_h);
  free(s_h);
  printf("ok\n");
  return 0;
}
