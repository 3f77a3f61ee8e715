// Launchers shared between the C ABI front end and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

constexpr int kSrcBf16 = 0;
constexpr int kSrcF32 = 1;

constexpr int kOutF32 = 0;
constexpr int kOutBf16 = 1;
constexpr int kOutMx = 2;

constexpr int kLayoutRows = 0;
constexpr int kLayoutTiled = 1;

// Element formats; the values are the format codes of the gfx950 scaled
// f8f6f4 MFMA instructions.
constexpr int kFmtE4M3 = 0;
constexpr int kFmtE5M2 = 1;
constexpr int kFmtE2M3 = 2;
constexpr int kFmtE3M2 = 3;
constexpr int kFmtE2M1 = 4;

// Bits per element code: a 32-element block is 4 * bits bytes, and the
// block's codes fill `bits` dwords.
constexpr int fmt_bits(int fmt) { return fmt == kFmtE2M1 ? 4 : (fmt == kFmtE4M3 || fmt == kFmtE5M2) ? 8 : 6; }

// Tiled MX layout: 128-element stages x 32-row groups, 512 * bits code bytes
// (3072 for the 6-bit types) and 128 scale bytes per (stage, group).
constexpr int kTileStageK = 128;
constexpr int kTileGroupRows = 32;
constexpr int kChunkCodes = 3072;
constexpr int kChunkScales = 128;
constexpr int chunk_codes(int bits) { return 512 * bits; }
constexpr int half_codes(int bits) { return 256 * bits; }
// Planes of one half (blocks 2h and 2h+1 of a stage, 32 rows) of a tiled chunk:
// A = bytes 0..15 of block 2h (16 per row), L = its bytes 16..23 (8 per row),
// H = bytes 0..7 of block 2h+1 (8 per row), B = its bytes 8..23 (16 per row).
constexpr int kHalfBytes = 1536;
constexpr int kPlaneA = 0;
constexpr int kPlaneL = 512;
constexpr int kPlaneH = 768;
constexpr int kPlaneB = 1024;
// 8-bit types: four planes of 16 bytes per row in each 2048-byte half h:
// bytes 16h..16h+15 of blocks 0, 2, 1, 3 (plane 2s + r holds block 2r + s).
// 4-bit types: two planes of 16 bytes per row in each 1024-byte half: block
// 2h, then block 2h+1.
constexpr int kPlaneStride16 = 512;  // one plane of 32 rows x 16 bytes

constexpr int kEpiNone = 0;
constexpr int kEpiGeluTanh = 1;
constexpr int kEpiSwiglu = 2;   // stacked gate/up rows (runs of 64 + 64), out[:, f] = silu(gate f) * up f

// Main GEMM tile: 256 tokens x 256 (or 128) output features, K staged 128 at a time.
constexpr int kTileM = 256;
constexpr int kStageK = 128;

struct GemmArgs {
  const uint8_t* x_codes;   // activations [M, K], tiled layout
  const uint8_t* x_scales;
  const uint8_t* w_codes;   // weights [N, K], tiled layout
  const uint8_t* w_scales;
  void* out;                // f32 / bf16 [M, ldo], or MX codes of [M, N] in the tiled layout
  uint8_t* out_scales;      // MX output scales (tiled layout)
  int64_t ldo;
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
  int32_t gx, gw;           // 32-row groups of the activations (ceil(M/32)) and weights (ceil(N/32))
  int32_t vec_store;        // 1 when 16-byte vector stores of a row segment are aligned
  int32_t group_m;          // tile order: m-tiles per group (1 .. 16)
  int32_t xcd_remap;        // tile order: 1 = contiguous tile ranges per XCD
  int32_t tile_n;           // output features per tile: 256 or 128
  int32_t waves;            // waves per workgroup: 4 or 8 (tile_n 256)
};

hipError_t launch_quantize(const void* src, int src_type, int64_t rows, int64_t k, int64_t ld_src, int fmt,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_quantize_tiled(const void* src, int src_type, int64_t rows, int64_t k, int64_t ld_src, int fmt,
                                 uint8_t* codes, uint8_t* scales, hipStream_t stream);

hipError_t launch_gemm(const GemmArgs& a, int x_fmt, int w_fmt, int epilogue, int out_kind, int out_fmt,
                       hipStream_t stream);

constexpr int kMaxSplits = 16;  // split-K chunks (their partials live in LDS)

struct SplitKArgs {
  const uint8_t* x_codes;   // activations [M, K], M <= 16, tiled layout (one 32-row group)
  const uint8_t* x_scales;
  const uint8_t* w_codes;   // weights [N, K], tiled layout
  const uint8_t* w_scales;
  void* out;                // f32 / bf16 [M, ldo]
  int64_t ldo;
  int32_t M, N, K, splits;
  int32_t gw;               // 32-row groups of the weights
};

hipError_t launch_gemm_splitk(const SplitKArgs& a, int x_fmt, int w_fmt, int out_kind, hipStream_t stream);

// RMSNorm + modulation + MX quantization into the tiled layout (one workgroup per 32-row group).
struct ProducerArgs {
  const void* x;            // bf16 / fp32 [rows, d], row r at x + r * ld_bytes
  int64_t ld_bytes;
  int32_t rows, d, groups;  // groups = ceil(rows / 32)
  const float* gamma;       // [d] or null (ones)
  const float* shift;       // [n_cond, d] or null (zeros)
  const float* scale;       // [n_cond, d] or null (zeros)
  int64_t rows_per_cond;    // a multiple of 32 (0 when shift and scale are null)
  float eps;
  uint8_t* codes;           // tiled layout of the [rows, d] output
  uint8_t* scales;
};

hipError_t launch_rmsnorm_quantize(const ProducerArgs& a, int src_type, int fmt, hipStream_t stream);

}  // namespace mxg

namespace mxg {
template <int WF, int XF>
hipError_t launch_gemm_formats(const GemmArgs& a, int epilogue, int out_kind, int out_fmt, hipStream_t stream);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t tiled_codes_bytes(int64_t rows, int64_t k, int bits) {
  return ceil_div(k, kTileStageK) * ceil_div(rows, kTileGroupRows) * chunk_codes(bits);
}
inline int64_t tiled_scales_bytes(int64_t rows, int64_t k) {
  return ceil_div(k, kTileStageK) * ceil_div(rows, kTileGroupRows) * kChunkScales;
}
}  // namespace mxg
