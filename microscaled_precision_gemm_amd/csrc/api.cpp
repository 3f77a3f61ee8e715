// C ABI front end: argument validation on the host (before any HIP call),
// workspace layout and kernel dispatch.  See include/mxgemm.h for the contract.
#include "mxgemm.h"

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "grid_limits.h"
#include "internal.h"
#include "mx_device.h"

// ---- the allocation-free split-K entry point's scratch.  The activations
// that mx_gemm_splitk_noalloc quantizes inside the call go to this
// file-scope device array instead of a caller workspace: at most 16 rows
// (one 32-row group of the tiled layout) of k <= MX_NOALLOC_MAX_K 6-bit
// codes and their scales.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code the array's name only stands in for
// the symbol: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and that pointer is what
// the kernels receive.  The quantizer rewrites every byte the GEMM reads
// (padding included) on each call, so nothing needs clearing between calls.
constexpr size_t kNoAllocScratchBytes =
    (size_t)(MX_NOALLOC_MAX_K / 128) * 3072 + (size_t)(MX_NOALLOC_MAX_K / 128) * 128;  // codes, then scales
static_assert((MX_NOALLOC_MAX_K / 128) * 3072 % 256 == 0, "the scales start 256-byte aligned, as in a workspace");
static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];

namespace {

using namespace mxg;

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr size_t kWsAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_fmt(int32_t f) {
  return f == MX_FMT_E2M3 || f == MX_FMT_E3M2 || f == MX_FMT_E2M1 || f == MX_FMT_E4M3 || f == MX_FMT_E5M2;
}

bool fp6_fmt(int32_t f) { return f == MX_FMT_E2M3 || f == MX_FMT_E3M2; }

int hip_status(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

// Launch log: with MXGEMM_LOG=1 in the environment (read once), every call of
// a computing entry point writes one line to stderr: the call, its sizes,
// formats and options, and the status it returns.  Off by default.
bool log_on() {
  static const bool on = [] {
    const char* e = getenv("MXGEMM_LOG");
    return e != nullptr && e[0] == '1' && e[1] == '\0';
  }();
  return on;
}

__attribute__((format(printf, 2, 3))) int logged(int status, const char* fmt, ...) {
  if (log_on()) {
    char line[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(line, sizeof line, fmt, ap);
    va_end(ap);
    fprintf(stderr, "mxgemm: %s -> %d (%s)\n", line, status, mx_status_string(status));
  }
  return status;
}

bool valid_layout(int32_t l) { return l == MX_LAYOUT_ROWS || l == MX_LAYOUT_TILED; }

int check_quantize_args(const void* src, int32_t src_type, int64_t rows, int64_t k, int64_t ld_src, int32_t fmt,
                        int32_t layout, const void* codes, const void* scales) {
  if (src_type != MX_SRC_BF16 && src_type != MX_SRC_F32) return MX_ERR_FORMAT;
  if (!valid_fmt(fmt) || !valid_layout(layout)) return MX_ERR_FORMAT;
  if (rows < 0 || k < 0 || k % 32 != 0 || rows > kMaxDim || k > kMaxDim) return MX_ERR_SHAPE;
  if (rows == 0 || k == 0) return MX_OK;
  if (!src || !codes || !scales) return MX_ERR_NULL;
  if (ld_src < k || ld_src > kMaxDim) return MX_ERR_SHAPE;
  const int64_t esize = src_type == MX_SRC_BF16 ? 2 : 4;
  if (!aligned(src, 16) || (ld_src * esize) % 16 != 0) return MX_ERR_ALIGN;
  if (!aligned(codes, 16) || !aligned(scales, 4)) return MX_ERR_ALIGN;
  return MX_OK;
}

// Workspace for activations quantized inside mx_gemm: tiled codes then
// scales.  Its advertised size is the one of 8-bit codes, which covers every
// element format.
struct TiledWs {
  size_t codes_off, scales_off, end;
};

TiledWs tiled_ws(int64_t rows, int64_t k, int bits) {
  TiledWs w;
  w.codes_off = 0;
  w.scales_off = round_up((size_t)tiled_codes_bytes(rows, k, bits), kWsAlign);
  w.end = w.scales_off + round_up((size_t)tiled_scales_bytes(rows, k), kWsAlign);
  return w;
}

// Common checks of the GEMM operands; fills the quantized-activation pointers.
int check_gemm_common(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes, const uint8_t* a_scales,
                      int32_t a_fmt, const void* w_codes, const uint8_t* w_scales, int32_t w_fmt, int64_t m, int64_t n,
                      int64_t k) {
  if (m < 0 || n < 0 || k < 0 || k % 32 != 0 || m > kMaxDim || n > kMaxDim || k > kMaxDim) return MX_ERR_SHAPE;
  if (!valid_fmt(a_fmt) || !valid_fmt(w_fmt)) return MX_ERR_FORMAT;
  // The scaled MFMA loses fp32 accuracy when both operands are E3M2 (measured on
  // gfx950: errors up to ~4e-5 of sum|a*b|), which breaks the GEMM tolerance.
  if (a_fmt == MX_FMT_E3M2 && w_fmt == MX_FMT_E3M2) return MX_ERR_UNSUPPORTED;
  // kernel variants: the 6-bit pairs above, E2M1 x E2M1, and 8-bit x 8-bit
  const int ba = fmt_bits(a_fmt), bw = fmt_bits(w_fmt);
  if (ba != bw) return MX_ERR_UNSUPPORTED;
  if (k == 0) {
    // nothing is read: C = 0; empty operands may come with NULL pointers
    if (a_src && a_src_type != MX_SRC_BF16 && a_src_type != MX_SRC_F32) return MX_ERR_FORMAT;
    return MX_OK;
  }
  if ((a_src != nullptr) == (a_codes != nullptr)) return MX_ERR_NULL;  // exactly one activation form
  if (a_src) {
    if (a_src_type != MX_SRC_BF16 && a_src_type != MX_SRC_F32) return MX_ERR_FORMAT;
    if (lda < k || lda > kMaxDim) return MX_ERR_SHAPE;
    const int64_t esize = a_src_type == MX_SRC_BF16 ? 2 : 4;
    if (!aligned(a_src, 16) || (lda * esize) % 16 != 0) return MX_ERR_ALIGN;
  } else {
    if (!a_scales) return MX_ERR_NULL;
    if (!aligned(a_codes, 16) || !aligned(a_scales, 4)) return MX_ERR_ALIGN;
  }
  if (!w_codes || !w_scales) return MX_ERR_NULL;
  if (!aligned(w_codes, 16) || !aligned(w_scales, 4)) return MX_ERR_ALIGN;
  return MX_OK;
}

// mx_gemm_splitk's host-side checks (everything but the workspace).
int check_splitk(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes, const uint8_t* a_scales,
                 int32_t a_fmt, const void* w_codes, const uint8_t* w_scales, int32_t w_fmt, int64_t m, int64_t n,
                 int64_t k, int32_t splits, int32_t out_kind, const void* out, int64_t ldo) {
  int st = check_gemm_common(a_src, a_src_type, lda, a_codes, a_scales, a_fmt, w_codes, w_scales, w_fmt, m, n, k);
  if (st != MX_OK) return st;
  if (m > 16) return MX_ERR_SHAPE;
  if (splits < 1) return MX_ERR_SHAPE;
  if (!fp6_fmt(a_fmt) || !fp6_fmt(w_fmt)) return MX_ERR_UNSUPPORTED;
  if (out_kind != MX_OUT_F32 && out_kind != MX_OUT_BF16) return MX_ERR_FORMAT;
  if (!out) return MX_ERR_NULL;
  if (ldo < n || ldo > kMaxDim) return MX_ERR_SHAPE;
  if (!aligned(out, out_kind == MX_OUT_F32 ? 4 : 2)) return MX_ERR_ALIGN;
  if (splits > kMaxSplits || k % (kTileStageK * (int64_t)splits) != 0) return MX_ERR_UNSUPPORTED;
  if (splitk_grid_items(n) > kMaxGridItems) return MX_ERR_UNSUPPORTED;
  return MX_OK;
}

// The split-K launch after validation: in-call quantization into ws (when
// a_src is given), then the split-K kernel.
int run_splitk(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes, const uint8_t* a_scales,
               int32_t a_fmt, const void* w_codes, const uint8_t* w_scales, int32_t w_fmt, int64_t m, int64_t n,
               int64_t k, int32_t splits, int32_t out_kind, void* out, int64_t ldo, uint8_t* ws, hipStream_t stream) {
  const uint8_t* xc = static_cast<const uint8_t*>(a_codes);
  const uint8_t* xs = a_scales;
  if (a_src && k > 0) {
    const TiledWs w = tiled_ws(m, k, 6);
    const hipError_t e =
        launch_quantize_tiled(a_src, a_src_type, m, k, lda, a_fmt, ws + w.codes_off, ws + w.scales_off, stream);
    if (e != hipSuccess) return MX_ERR_HIP;
    xc = ws + w.codes_off;
    xs = ws + w.scales_off;
  }
  SplitKArgs g;
  g.x_codes = xc;
  g.x_scales = xs;
  g.w_codes = static_cast<const uint8_t*>(w_codes);
  g.w_scales = w_scales;
  g.out = out;
  g.ldo = ldo;
  g.M = (int32_t)m;
  g.N = (int32_t)n;
  g.K = (int32_t)k;
  g.splits = splits;
  g.gw = (int32_t)ceil_div(n, kTileGroupRows);
  return hip_status(launch_gemm_splitk(g, a_fmt, w_fmt, out_kind, stream));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MX_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MX_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MX_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MX_OK;
}

}  // namespace

namespace mxg {
hipError_t launch_gemm(const GemmArgs& a, int x_fmt, int w_fmt, int epilogue, int out_kind, int out_fmt,
                       hipStream_t stream) {
  if (w_fmt == kFmtE2M3 && x_fmt == kFmtE2M3) return launch_gemm_formats<kFmtE2M3, kFmtE2M3>(a, epilogue, out_kind, out_fmt, stream);
  if (w_fmt == kFmtE3M2 && x_fmt == kFmtE2M3) return launch_gemm_formats<kFmtE3M2, kFmtE2M3>(a, epilogue, out_kind, out_fmt, stream);
  if (w_fmt == kFmtE2M3 && x_fmt == kFmtE3M2) return launch_gemm_formats<kFmtE2M3, kFmtE3M2>(a, epilogue, out_kind, out_fmt, stream);
  if (w_fmt == kFmtE2M1 && x_fmt == kFmtE2M1) return launch_gemm_formats<kFmtE2M1, kFmtE2M1>(a, epilogue, out_kind, out_fmt, stream);
  if (w_fmt == kFmtE4M3 && x_fmt == kFmtE4M3) return launch_gemm_formats<kFmtE4M3, kFmtE4M3>(a, epilogue, out_kind, out_fmt, stream);
  if (w_fmt == kFmtE5M2 && x_fmt == kFmtE5M2) return launch_gemm_formats<kFmtE5M2, kFmtE5M2>(a, epilogue, out_kind, out_fmt, stream);
  if (w_fmt == kFmtE4M3 && x_fmt == kFmtE5M2) return launch_gemm_formats<kFmtE4M3, kFmtE5M2>(a, epilogue, out_kind, out_fmt, stream);
  if (w_fmt == kFmtE5M2 && x_fmt == kFmtE4M3) return launch_gemm_formats<kFmtE5M2, kFmtE4M3>(a, epilogue, out_kind, out_fmt, stream);
  return hipErrorInvalidValue;  // other pairs are rejected before this point
}
}  // namespace mxg

extern "C" {

int mx_version(void) { return 400; }

const char* mx_status_string(int status) {
  switch (status) {
    case MX_OK: return "ok";
    case MX_ERR_NULL: return "a required pointer is NULL (or both/neither activation forms given)";
    case MX_ERR_SHAPE: return "invalid size: negative, too large, K not a multiple of 32, or leading dimension too small";
    case MX_ERR_FORMAT: return "unknown element format, source type, output kind or epilogue";
    case MX_ERR_ALIGN: return "a pointer or leading dimension is not aligned as required";
    case MX_ERR_WORKSPACE: return "workspace missing or smaller than mx_gemm_workspace_size()";
    case MX_ERR_UNSUPPORTED: return "valid request without a kernel variant";
    case MX_ERR_HIP: return "HIP kernel launch failed";
    case MX_ERR_SCRATCH:
      return "request larger than the static scratch of mx_gemm_splitk_noalloc (k > MX_NOALLOC_MAX_K)";
    default: return "unknown status";
  }
}

static int rmsnorm_quantize_call(const void* x, int32_t src_type, int64_t rows, int64_t d, int64_t ld_x, const float* gamma,
                        const float* shift, const float* scale, int64_t rows_per_cond, float eps, int32_t fmt,
                        void* codes, uint8_t* scales, hipStream_t stream) {
  int st = check_quantize_args(x, src_type, rows, d, ld_x, fmt, MX_LAYOUT_TILED, codes, scales);
  if (st != MX_OK) return st;
  if (!fp6_fmt(fmt)) return MX_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return MX_ERR_SHAPE;  // rejects NaN, negative and infinite eps
  const bool modulated = shift != nullptr || scale != nullptr;
  if (modulated && (rows_per_cond <= 0 || rows_per_cond % 32 != 0)) return MX_ERR_SHAPE;
  if (rows == 0 || d == 0) return MX_OK;
  if (!aligned(gamma, 4) || !aligned(shift, 4) || !aligned(scale, 4)) return MX_ERR_ALIGN;
  if (tiled_codes_bytes(rows, d, 6) >= ((int64_t)1 << 40)) return MX_ERR_UNSUPPORTED;
  if (rmsnorm_quantize_grid_items(rows, d, src_type == MX_SRC_F32 ? kSrcF32 : kSrcBf16) > kMaxGridItems)
    return MX_ERR_UNSUPPORTED;
  ProducerArgs a;
  a.x = x;
  a.ld_bytes = ld_x * (src_type == MX_SRC_BF16 ? 2 : 4);
  a.rows = (int32_t)rows;
  a.d = (int32_t)d;
  a.groups = (int32_t)ceil_div(rows, kTileGroupRows);
  a.gamma = gamma;
  a.shift = shift;
  a.scale = scale;
  a.rows_per_cond = modulated ? rows_per_cond : 0;
  a.eps = eps;
  a.codes = static_cast<uint8_t*>(codes);
  a.scales = scales;
  return hip_status(launch_rmsnorm_quantize(a, src_type, fmt, stream));
}

size_t mx_packed_bytes(int64_t rows, int64_t k, int32_t fmt, int32_t layout, int32_t which) {
  if (rows < 0 || k < 0 || k % 32 != 0 || rows > kMaxDim || k > kMaxDim || !valid_layout(layout)) return 0;
  if (!valid_fmt(fmt) || (which != 0 && which != 1)) return 0;
  const int bits = fmt_bits(fmt);
  if (layout == MX_LAYOUT_ROWS) return (size_t)(which == 0 ? rows * (k / 32) * 4 * bits : rows * (k / 32));
  return (size_t)(which == 0 ? tiled_codes_bytes(rows, k, bits) : tiled_scales_bytes(rows, k));
}

size_t mx_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int32_t a_is_src, int32_t splits) {
  if (m < 0 || n < 0 || k < 0 || k % 32 != 0 || m > kMaxDim || n > kMaxDim || k > kMaxDim || splits < 0) return 0;
  if (splits == 0) return a_is_src ? tiled_ws(m, k, 8).end : 0;
  if (m > 16 || splits > kMaxSplits) return 0;
  return a_is_src ? tiled_ws(m, k, 8).end : 0;
}

static int quantize_call(const void* src, int32_t src_type, int64_t rows, int64_t k, int64_t ld_src, int32_t fmt,
                int32_t layout, void* codes, uint8_t* scales, hipStream_t stream) {
  const int st = check_quantize_args(src, src_type, rows, k, ld_src, fmt, layout, codes, scales);
  if (st != MX_OK || rows == 0 || k == 0) return st;
  if (quantize_grid_items(rows, k, layout == MX_LAYOUT_TILED ? kLayoutTiled : kLayoutRows) > kMaxGridItems)
    return MX_ERR_UNSUPPORTED;
  if (layout == MX_LAYOUT_TILED) {
    if (tiled_codes_bytes(rows, k, fmt_bits(fmt)) >= ((int64_t)1 << 40)) return MX_ERR_UNSUPPORTED;
    return hip_status(
        launch_quantize_tiled(src, src_type, rows, k, ld_src, fmt, static_cast<uint8_t*>(codes), scales, stream));
  }
  return hip_status(launch_quantize(src, src_type, rows, k, ld_src, fmt, static_cast<uint8_t*>(codes), scales, stream));
}

void mx_gemm_default_config(mx_gemm_config* config) {
  if (!config) return;
  config->group_m = 4;
  config->xcd_remap = 1;
  config->tile_n = 256;
  config->waves = 4;
}

void mx_gemm_select_config(int64_t m, int64_t n, int64_t k, int32_t a_fmt, int32_t w_fmt, int32_t epilogue,
                           int32_t out_kind, mx_gemm_config* config) {
  if (!config) return;
  mx_gemm_default_config(config);
  (void)m;
  (void)n;
  const bool fp8 = fmt_bits(a_fmt) == 8 || fmt_bits(w_fmt) == 8;
  if (fp8) return;  // 8 waves slow FP8 down (two ring slots at 8 bits)
  // the 4- and 6-bit types: two waves per SIMD hide the operand reads from
  // LDS behind the other wave's matrix work; with the GELU / identity MX
  // epilogue (fc1's shape) a wider tile walk as well
  config->waves = 8;
  if (out_kind == MX_OUT_MX && epilogue != MX_EPI_SWIGLU) config->group_m = 8;
}

int mx_gemm(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes, const uint8_t* a_scales,
            int32_t a_fmt, const void* w_codes, const uint8_t* w_scales, int32_t w_fmt, int64_t m, int64_t n, int64_t k,
            int32_t epilogue, int32_t out_kind, void* out, int64_t ldo, uint8_t* out_scales, int32_t out_fmt,
            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return mx_gemm_with_config(a_src, a_src_type, lda, a_codes, a_scales, a_fmt, w_codes, w_scales, w_fmt, m, n, k,
                             epilogue, out_kind, out, ldo, out_scales, out_fmt, workspace, workspace_bytes, nullptr,
                             stream);
}

static int gemm_call(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes,
                        const uint8_t* a_scales, int32_t a_fmt, const void* w_codes, const uint8_t* w_scales,
                        int32_t w_fmt, int64_t m, int64_t n, int64_t k, int32_t epilogue, int32_t out_kind, void* out,
                        int64_t ldo, uint8_t* out_scales, int32_t out_fmt, void* workspace, size_t workspace_bytes,
                        const mx_gemm_config* config, hipStream_t stream) {
  mx_gemm_config cfg;
  mx_gemm_select_config(m, n, k, a_fmt, w_fmt, epilogue, out_kind, &cfg);
  if (config) {
    if (config->group_m < 1 || config->group_m > 16 || (config->xcd_remap != 0 && config->xcd_remap != 1) ||
        (config->tile_n != 256 && config->tile_n != 128) || (config->waves != 4 && config->waves != 8))
      return MX_ERR_FORMAT;
    cfg = *config;
  }
  int st = check_gemm_common(a_src, a_src_type, lda, a_codes, a_scales, a_fmt, w_codes, w_scales, w_fmt, m, n, k);
  if (st != MX_OK) return st;
  if (epilogue != MX_EPI_NONE && epilogue != MX_EPI_GELU_TANH && epilogue != MX_EPI_SWIGLU) return MX_ERR_FORMAT;
  if (out_kind != MX_OUT_F32 && out_kind != MX_OUT_BF16 && out_kind != MX_OUT_MX) return MX_ERR_FORMAT;
  // SwiGLU pairs the gate and up rows inside each run of 128 stacked rows
  if (epilogue == MX_EPI_SWIGLU && n % 128 != 0) return MX_ERR_UNSUPPORTED;
  // the 4- and 8-bit operand formats have the plain product with fp32 / bf16 output
  if (!fp6_fmt(w_fmt) && (epilogue != MX_EPI_NONE || out_kind == MX_OUT_MX)) return MX_ERR_UNSUPPORTED;
  // 128-feature tiles: the 6-bit pairs
  if (cfg.tile_n == 128 && !fp6_fmt(w_fmt)) return MX_ERR_UNSUPPORTED;
  // eight waves: 256-feature tiles
  if (cfg.waves == 8 && cfg.tile_n != 256) return MX_ERR_UNSUPPORTED;
  const int64_t n_out = epilogue == MX_EPI_SWIGLU ? n / 2 : n;
  if (!out) return MX_ERR_NULL;
  if (out_kind == MX_OUT_MX) {
    if (!valid_fmt(out_fmt)) return MX_ERR_FORMAT;
    if (!fp6_fmt(out_fmt)) return MX_ERR_UNSUPPORTED;
    if (!out_scales) return MX_ERR_NULL;
    if (n_out % 32 != 0) return MX_ERR_UNSUPPORTED;
    if (!aligned(out, 16) || !aligned(out_scales, 4)) return MX_ERR_ALIGN;
  } else {
    if (ldo < n_out || ldo > kMaxDim) return MX_ERR_SHAPE;
    if (!aligned(out, out_kind == MX_OUT_F32 ? 4 : 2)) return MX_ERR_ALIGN;
  }
  const size_t need = mx_gemm_workspace_size(m, n, k, a_src != nullptr, 0);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MX_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, kWsAlign)) return MX_ERR_ALIGN;
  if (m == 0 || n == 0) return MX_OK;
  // launch limits, checked before anything is launched
  const int64_t tiles_m = ceil_div(m, kTileM), tiles_n = ceil_div(n, cfg.tile_n);
  if (tiles_m * tiles_n > INT32_MAX) return MX_ERR_SHAPE;
  if (gemm_grid_items(tiles_m, tiles_n, cfg.waves) > kMaxGridItems) return MX_ERR_UNSUPPORTED;
  // the kernel addresses one stage of an operand with 32-bit offsets
  const int64_t chunk = chunk_codes(fmt_bits(w_fmt));
  if (ceil_div(m, kTileGroupRows) * chunk >= ((int64_t)1 << 32) || ceil_div(n, kTileGroupRows) * chunk >= ((int64_t)1 << 32))
    return MX_ERR_UNSUPPORTED;

  const uint8_t* xc = static_cast<const uint8_t*>(a_codes);
  const uint8_t* xs = a_scales;
  if (a_src && k > 0) {
    const TiledWs w = tiled_ws(m, k, fmt_bits(a_fmt));
    uint8_t* base = static_cast<uint8_t*>(workspace);
    const hipError_t e = launch_quantize_tiled(a_src, a_src_type, m, k, lda, a_fmt, base + w.codes_off,
                                               base + w.scales_off, stream);
    if (e != hipSuccess) return MX_ERR_HIP;
    xc = base + w.codes_off;
    xs = base + w.scales_off;
  }
  GemmArgs g;
  g.x_codes = xc;
  g.x_scales = xs;
  g.w_codes = static_cast<const uint8_t*>(w_codes);
  g.w_scales = w_scales;
  g.out = out;
  g.out_scales = out_scales;
  g.ldo = ldo;
  g.M = (int32_t)m;
  g.N = (int32_t)n;
  g.K = (int32_t)k;
  g.tiles_m = (int32_t)tiles_m;
  g.tiles_n = (int32_t)tiles_n;
  g.tile_n = cfg.tile_n;
  g.waves = cfg.waves;
  g.gx = (int32_t)ceil_div(m, kTileGroupRows);
  g.gw = (int32_t)ceil_div(n, kTileGroupRows);
  const int64_t esize = out_kind == MX_OUT_F32 ? 4 : 2;
  g.vec_store = out_kind != MX_OUT_MX && aligned(out, 16) && (ldo * esize) % 16 == 0;
  g.group_m = cfg.group_m;
  g.xcd_remap = cfg.xcd_remap;
  return hip_status(launch_gemm(g, a_fmt, w_fmt, epilogue, out_kind, out_fmt, stream));
}

static int splitk_call(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes, const uint8_t* a_scales,
                   int32_t a_fmt, const void* w_codes, const uint8_t* w_scales, int32_t w_fmt, int64_t m, int64_t n,
                   int64_t k, int32_t splits, int32_t out_kind, void* out, int64_t ldo, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  int st = check_splitk(a_src, a_src_type, lda, a_codes, a_scales, a_fmt, w_codes, w_scales, w_fmt, m, n, k, splits,
                        out_kind, out, ldo);
  if (st != MX_OK) return st;
  const size_t need = mx_gemm_workspace_size(m, n, k, a_src != nullptr, splits);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MX_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, kWsAlign)) return MX_ERR_ALIGN;
  if (m == 0 || n == 0) return MX_OK;
  return run_splitk(a_src, a_src_type, lda, a_codes, a_scales, a_fmt, w_codes, w_scales, w_fmt, m, n, k, splits,
                    out_kind, out, ldo, static_cast<uint8_t*>(workspace), stream);
}

static int splitk_noalloc_call(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes,
                           const uint8_t* a_scales, int32_t a_fmt, const void* w_codes, const uint8_t* w_scales,
                           int32_t w_fmt, int64_t m, int64_t n, int64_t k, int32_t splits, int32_t out_kind,
                           void* out, int64_t ldo, hipStream_t stream) {
  int st = check_splitk(a_src, a_src_type, lda, a_codes, a_scales, a_fmt, w_codes, w_scales, w_fmt, m, n, k, splits,
                        out_kind, out, ldo);
  if (st != MX_OK) return st;
  if (k > MX_NOALLOC_MAX_K) return MX_ERR_SCRATCH;
  // what run_splitk writes: one 32-row group of 6-bit codes, then scales
  if (a_src && tiled_ws(m, k, 6).end > kNoAllocScratchBytes) return MX_ERR_SCRATCH;
  if (m == 0 || n == 0) return MX_OK;
  uint8_t* ws = nullptr;
  if (a_src && k > 0) {
    st = noalloc_scratch(&ws);
    if (st != MX_OK) return st;
  }
  return run_splitk(a_src, a_src_type, lda, a_codes, a_scales, a_fmt, w_codes, w_scales, w_fmt, m, n, k, splits,
                    out_kind, out, ldo, ws, stream);
}

// ---- the computing entry points: the calls above plus the launch log

int mx_quantize(const void* src, int32_t src_type, int64_t rows, int64_t k, int64_t ld_src, int32_t fmt,
                int32_t layout, void* codes, uint8_t* scales, hipStream_t stream) {
  return logged(quantize_call(src, src_type, rows, k, ld_src, fmt, layout, codes, scales, stream),
                "mx_quantize rows=%lld k=%lld ld=%lld src_type=%d fmt=%d layout=%d", (long long)rows, (long long)k,
                (long long)ld_src, src_type, fmt, layout);
}

int mx_rmsnorm_quantize(const void* x, int32_t src_type, int64_t rows, int64_t d, int64_t ld_x, const float* gamma,
                        const float* shift, const float* scale, int64_t rows_per_cond, float eps, int32_t fmt,
                        void* codes, uint8_t* scales, hipStream_t stream) {
  return logged(rmsnorm_quantize_call(x, src_type, rows, d, ld_x, gamma, shift, scale, rows_per_cond, eps, fmt, codes,
                                      scales, stream),
                "mx_rmsnorm_quantize rows=%lld d=%lld ld=%lld src_type=%d fmt=%d gamma=%d shift=%d scale=%d "
                "rows_per_cond=%lld eps=%g",
                (long long)rows, (long long)d, (long long)ld_x, src_type, fmt, gamma != nullptr, shift != nullptr,
                scale != nullptr, (long long)rows_per_cond, (double)eps);
}

int mx_gemm_with_config(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes,
                        const uint8_t* a_scales, int32_t a_fmt, const void* w_codes, const uint8_t* w_scales,
                        int32_t w_fmt, int64_t m, int64_t n, int64_t k, int32_t epilogue, int32_t out_kind, void* out,
                        int64_t ldo, uint8_t* out_scales, int32_t out_fmt, void* workspace, size_t workspace_bytes,
                        const mx_gemm_config* config, hipStream_t stream) {
  mx_gemm_config used;
  if (config)
    used = *config;
  else
    mx_gemm_select_config(m, n, k, a_fmt, w_fmt, epilogue, out_kind, &used);
  return logged(gemm_call(a_src, a_src_type, lda, a_codes, a_scales, a_fmt, w_codes, w_scales, w_fmt, m, n, k,
                          epilogue, out_kind, out, ldo, out_scales, out_fmt, workspace, workspace_bytes, config,
                          stream),
                "mx_gemm m=%lld n=%lld k=%lld a=%s fmt=%d w_fmt=%d epilogue=%d out_kind=%d out_fmt=%d "
                "config=(%d,%d,%d,%d)%s",
                (long long)m, (long long)n, (long long)k, a_src ? "src" : "mx", a_fmt, w_fmt, epilogue, out_kind,
                out_fmt, used.group_m, used.xcd_remap, used.tile_n, used.waves, config ? "" : " by shape rule");
}

int mx_gemm_splitk(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes, const uint8_t* a_scales,
                   int32_t a_fmt, const void* w_codes, const uint8_t* w_scales, int32_t w_fmt, int64_t m, int64_t n,
                   int64_t k, int32_t splits, int32_t out_kind, void* out, int64_t ldo, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  return logged(splitk_call(a_src, a_src_type, lda, a_codes, a_scales, a_fmt, w_codes, w_scales, w_fmt, m, n, k,
                            splits, out_kind, out, ldo, workspace, workspace_bytes, stream),
                "mx_gemm_splitk m=%lld n=%lld k=%lld a=%s fmt=%d w_fmt=%d splits=%d out_kind=%d", (long long)m,
                (long long)n, (long long)k, a_src ? "src" : "mx", a_fmt, w_fmt, splits, out_kind);
}

int mx_gemm_splitk_noalloc(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes,
                           const uint8_t* a_scales, int32_t a_fmt, const void* w_codes, const uint8_t* w_scales,
                           int32_t w_fmt, int64_t m, int64_t n, int64_t k, int32_t splits, int32_t out_kind,
                           void* out, int64_t ldo, hipStream_t stream) {
  return logged(splitk_noalloc_call(a_src, a_src_type, lda, a_codes, a_scales, a_fmt, w_codes, w_scales, w_fmt, m, n,
                                    k, splits, out_kind, out, ldo, stream),
                "mx_gemm_splitk_noalloc m=%lld n=%lld k=%lld a=%s fmt=%d w_fmt=%d splits=%d out_kind=%d",
                (long long)m, (long long)n, (long long)k, a_src ? "src" : "mx", a_fmt, w_fmt, splits, out_kind);
}

}  // extern "C"
