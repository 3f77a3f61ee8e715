/* The C ABI used from plain C99 (no C++, no Python, no GPU): the header
 * compiles as C, the library links, and the calls that need no device answer
 * as the header says.  Built and run by tests/test_abi.py; prints one line per
 * check and exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "mxgemm.h"

static int failures = 0;

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) failures++;
}

int main(void) {
  check(mx_version() == 400, "mx_version");
  check(strstr(mx_status_string(MX_ERR_SHAPE), "size") != NULL, "mx_status_string(MX_ERR_SHAPE)");
  check(strcmp(mx_status_string(-99), "unknown status") == 0, "mx_status_string(unknown)");

  /* tiled E2M3 [300, 416]: 4 stages x 10 row groups of 3072 code bytes and 128 scale bytes */
  check(mx_packed_bytes(300, 416, MX_FMT_E2M3, MX_LAYOUT_TILED, 0) == (size_t)4 * 10 * 3072, "packed codes");
  check(mx_packed_bytes(300, 416, MX_FMT_E2M3, MX_LAYOUT_TILED, 1) == (size_t)4 * 10 * 128, "packed scales");
  check(mx_packed_bytes(300, 416, MX_FMT_E2M3, MX_LAYOUT_ROWS, 0) == (size_t)300 * 416 * 3 / 4, "rows codes");

  mx_gemm_config c;
  mx_gemm_default_config(&c);
  check(c.group_m == 4 && c.xcd_remap == 1 && c.tile_n == 256 && c.waves == 4, "default config");
  mx_gemm_select_config(20480, 12288, 3072, MX_FMT_E2M3, MX_FMT_E2M3, MX_EPI_GELU_TANH, MX_OUT_MX, &c);
  check(c.tile_n == 256 && c.waves == 8 && c.group_m == 8, "shape rule, fc1");

  check(mx_gemm_workspace_size(64, 64, 128, 0, 0) == 0, "no workspace for quantized activations");
  check(mx_gemm_workspace_size(16, 13312, 16384, 1, 16) > 0, "split-K workspace for bf16 activations");

  /* argument errors come back before anything touches a pointer or the GPU */
  check(mx_quantize(NULL, MX_SRC_BF16, 4, 48, 48, MX_FMT_E2M3, MX_LAYOUT_TILED, NULL, NULL, NULL) == MX_ERR_SHAPE,
        "mx_quantize: K not a multiple of 32");
  check(mx_quantize(NULL, 9, 4, 64, 64, MX_FMT_E2M3, MX_LAYOUT_TILED, NULL, NULL, NULL) == MX_ERR_FORMAT,
        "mx_quantize: unknown source type");
  check(mx_quantize(NULL, MX_SRC_BF16, 0, 64, 64, MX_FMT_E2M3, MX_LAYOUT_TILED, NULL, NULL, NULL) == MX_OK,
        "mx_quantize: empty is a no-op");
  check(mx_gemm(NULL, MX_SRC_BF16, 0, NULL, NULL, MX_FMT_E3M2, NULL, NULL, MX_FMT_E3M2, 64, 64, 128, MX_EPI_NONE,
                MX_OUT_BF16, NULL, 64, NULL, MX_FMT_E2M3, NULL, 0, NULL) == MX_ERR_UNSUPPORTED,
        "mx_gemm: E3M2 x E3M2");
  /* K = 0 reads no operand, so the pointers are not checked and the row count is */
  check(mx_gemm_splitk(NULL, MX_SRC_BF16, 0, NULL, NULL, MX_FMT_E2M3, NULL, NULL, MX_FMT_E3M2, 17, 64, 0, 8,
                       MX_OUT_BF16, NULL, 64, NULL, 0, NULL) == MX_ERR_SHAPE,
        "mx_gemm_splitk: more than 16 rows");
  check(mx_rmsnorm_quantize(NULL, MX_SRC_BF16, 4, 100, 100, NULL, NULL, NULL, 0, 1e-6f, MX_FMT_E2M3, NULL, NULL,
                            NULL) == MX_ERR_SHAPE,
        "mx_rmsnorm_quantize: d not a multiple of 32");
  return failures == 0 ? 0 : 1;
}
