// bf16 / fp32 -> MX quantizer for gfx950: the 6-bit element types E2M3 and
// E3M2, and the 4- and 8-bit types E2M1, E4M3 and E5M2 that the same scaled
// matrix instruction consumes.
//
// Each wave quantizes 64 consecutive 32-element blocks (row-major order over
// [rows, K/32]).  HBM-bound (2 or 4 bytes in, 0.5 to 1 byte out per element),
// so the design is about full-width memory transactions:
//
//  * loads: the wave reads its blocks as 16-byte pieces with consecutive lanes
//    on consecutive pieces (the 128-bit coalesced loads of the page "Creating
//    Custom Kernels for the AMD MI300", section "Fused RMS Norm Kernel"), and
//    an LDS transpose hands each lane one whole block;
//  * per block: amax on the raw magnitude bits, the E8M0 scale from the
//    exponent bits, and the v_cvt_scalef32 conversions that round the 32
//    elements (round-to-nearest-even, saturating, sign kept): one instruction
//    for a 6-bit block, 16 two-element ones for a 4- or 8-bit block;
//  * stores: the 64 blocks' code bytes of a wave are contiguous in the output,
//    so they go back through LDS and leave as 16-byte stores of consecutive
//    lanes.
#include <algorithm>

#include "grid_limits.h"
#include "internal.h"
#include "mx_device.h"

namespace mxg {

namespace {

constexpr int kQThreads = 256;
constexpr int kQWaves = kQThreads / 64;
constexpr int kInRowB = 16 * 5;                  // one block's bf16 bytes (64) padded to 80 for the LDS read
constexpr int kInRowF = 16 * 9;                  // fp32 (128) padded to 144
constexpr int kOutBytes = 64 * 32;               // code bytes of one wave (at most 32 per block)

// The 32 source values of a block held as 4 (bf16) or 8 (fp32) 16-byte pieces
// -> fp32, element i in v[i].
template <bool F32>
__device__ __forceinline__ void block_to_f32(const u32x4* w, float (&v)[32]) {
#pragma unroll
  for (int i = 0; i < (F32 ? 8 : 4); ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (F32) {
        v[4 * i + e] = __uint_as_float(w[i][e]);
      } else {
        v[8 * i + 2 * e] = __uint_as_float(w[i][e] << 16);
        v[8 * i + 2 * e + 1] = __uint_as_float(w[i][e] & 0xffff0000u);
      }
    }
}

// Scale rule + conversion of one block given as 16-byte pieces.  The 6-bit
// types convert bf16 directly with the 32-element instruction; everything else
// goes through fp32 values.
template <int FMT, bool F32>
__device__ __forceinline__ uint32_t quantize_block(const u32x4* w, uint32_t (&q)[fmt_bits(FMT)]) {
  BlockScale s;
  if constexpr (!F32) {
    // bf16: amax of the magnitude bits, two halves per dword (bit order = value order)
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t a = w[i][j] & 0x7fff7fffu;
        u16x2 v;
        __builtin_memcpy(&v, &a, 4);
        m2 = __builtin_elementwise_max(m2, v);
      }
    s = scale_from_bf16_bits<FMT>(m2[0] > m2[1] ? m2[0] : m2[1]);
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; j += 2) amax = absmax2(amax, __uint_as_float(w[i][j]), __uint_as_float(w[i][j + 1]));
    s = scale_from_f32_bits<FMT>(__float_as_uint(amax));
  }
  if constexpr (!F32 && fmt_bits(FMT) == 6) {
    v32bf x;
    __builtin_memcpy(&x, w, 64);
    const v6u r = cvt_bf16x32<FMT>(x, s.scale);
#pragma unroll
    for (int i = 0; i < 6; ++i) q[i] = r[i];
  } else {
    float v[32];
    block_to_f32<F32>(w, v);
    cvt_block<FMT>(v, s.scale, q);
  }
  if (s.nonfinite) {
#pragma unroll
    for (int i = 0; i < fmt_bits(FMT); ++i) q[i] = 0u;
  }
  return s.byte;
}

template <bool F32>
struct QLayout {
  static constexpr int kPieces = F32 ? 8 : 4;    // 16-byte pieces per block
  static constexpr int kRow = F32 ? kInRowF : kInRowB;
  static constexpr int kWaveIn = 64 * kRow;
};

template <int FMT, bool F32>
__global__ __launch_bounds__(kQThreads) void quantize_kernel(const uint8_t* __restrict__ src, int64_t ld_bytes,
                                                             int64_t kblocks, int64_t total_blocks,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales, int vec_out) {
  using L = QLayout<F32>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_in[kQWaves * L::kWaveIn];
  __shared__ __attribute__((aligned(16))) uint8_t lds_out[kQWaves * kOutBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wave_first = ((int64_t)blockIdx.x * kQWaves + wave) * 64;
  if (wave_first >= total_blocks) return;  // whole wave idle: no barrier below is shared across waves
  uint8_t* in = lds_in + wave * L::kWaveIn;
  uint8_t* outb = lds_out + wave * kOutBytes;

  // ---- coalesced loads: piece p of the wave (p = 64 i + lane) is piece p % kPieces of block p / kPieces
#pragma unroll
  for (int i = 0; i < L::kPieces; ++i) {
    const int p = 64 * i + lane;
    const int blk = p / L::kPieces, piece = p % L::kPieces;
    const int64_t b = wave_first + blk;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (b < total_blocks) {
      const int64_t row = b / kblocks, kb = b - row * kblocks;
      v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          src + row * ld_bytes + kb * (F32 ? 128 : 64) + piece * 16));
    }
    *reinterpret_cast<u32x4*>(in + blk * L::kRow + piece * 16) = v;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

  // ---- one block per lane
  constexpr int kBits = fmt_bits(FMT), kEB = 4 * kBits;  // code dwords / bytes per block
  const int64_t b = wave_first + lane;
  u32x4 w[L::kPieces];
#pragma unroll
  for (int i = 0; i < L::kPieces; ++i) w[i] = *reinterpret_cast<const u32x4*>(in + lane * L::kRow + i * 16);
  uint32_t q[kBits];
  const uint32_t byte = quantize_block<FMT, F32>(w, q);
  if (b < total_blocks) scales[b] = (uint8_t)byte;

  // ---- stores: the wave's code bytes are contiguous at codes + kEB * wave_first
  const int nblk = (int)min((int64_t)64, total_blocks - wave_first);
  if (vec_out && nblk == 64) {
#pragma unroll
    for (int i = 0; i < kBits / 2; ++i)
      *reinterpret_cast<u32x2*>(outb + kEB * lane + 8 * i) = u32x2{q[2 * i], q[2 * i + 1]};
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    uint8_t* dst = codes + (int64_t)kEB * wave_first;
#pragma unroll
    for (int p = lane; p < 4 * kEB; p += 64)
      *reinterpret_cast<u32x4*>(dst + 16 * p) = *reinterpret_cast<const u32x4*>(outb + 16 * p);
  } else if (b < total_blocks) {
    u32x2* o = reinterpret_cast<u32x2*>(codes + kEB * b);
#pragma unroll
    for (int i = 0; i < kBits / 2; ++i) o[i] = u32x2{q[2 * i], q[2 * i + 1]};
  }
}

// ---- tiled layout: one wave per (stage, 32-row group) chunk of 32 rows x 128
// elements.  Loads: 256 (bf16) or 512 (fp32) contiguous bytes per row, 16 per
// lane, consecutive lanes on consecutive bytes.  Each lane then converts two
// blocks of one row (blocks 2h, 2h+1 for lane half h), whose code bytes fill
// that row's entries of the planes of half h: for the 6-bit types 48 bytes in
// four planes (the 32 lanes of a half write runs of 512, 256, 256 and 512
// contiguous bytes), for the 8- and 4-bit types 64 or 32 bytes in 16-byte
// planes (runs of 512 bytes; an 8-bit block is split between the two halves
// of the chunk, the order in which the matrix instruction takes 8-bit
// operands).  Rows >= rows and blocks >= K/32 are written as padding (codes
// 0, scale 127).
constexpr int kTWaves = 4;
// workgroups resident at once on gfx950: 256 CUs x 4 (the 34 KB LDS each allows)
constexpr int64_t kTResident = 256 * 4;

template <bool F32>
struct TLayout {
  static constexpr int kRowSrc = F32 ? 512 : 256;       // source bytes per row of a chunk
  static constexpr int kRow = kRowSrc + 16;             // padded LDS row (conflict-free 16-byte reads)
  static constexpr int kPieces = kRowSrc / 16;           // 16-byte pieces per row
  static constexpr int kCopies = 32 * kPieces / 64;      // load instructions per wave
  static constexpr int kBlockSrc = F32 ? 128 : 64;       // source bytes per 32-element block
};

template <int FMT, bool F32>
__global__ __launch_bounds__(kTWaves * 64) void quantize_tiled_kernel(const uint8_t* __restrict__ src,
                                                                      int64_t ld_bytes, int rows, int k,
                                                                      int groups, int nchunks,
                                                                      uint8_t* __restrict__ codes,
                                                                      uint8_t* __restrict__ scales) {
  using L = TLayout<F32>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kTWaves * 32 * L::kRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Each wave converts chunks work, work + nwaves, ... in the group-major order
  // (all stages of rows 32g .. 32g+31, then the next group), so the waves in
  // flight read long runs of each row.  The next chunk's loads are issued
  // before the current one is converted, so every wave keeps a chunk of loads
  // in flight: the grid holds only as many workgroups as are resident at once.
  const int nwaves = gridDim.x * kTWaves;
  int work = blockIdx.x * kTWaves + wave;
  if (work >= nchunks) return;  // wave-level only: no workgroup barrier below
  const int stages = nchunks / groups;
  uint8_t* in = lds + wave * 32 * L::kRow;
  const int kblocks = k / 32;
  constexpr int kBits = fmt_bits(FMT);
  const int j = lane & 31, h = lane >> 5;

  // loads of chunk `w` (group-major order) into registers
  auto load = [&](int w, u32x4 (&v)[L::kCopies]) {
    const int grp = w / stages, stage = w - grp * stages;
#pragma unroll
    for (int i = 0; i < L::kCopies; ++i) {
      const int c = 64 * i + lane;
      const int jr = c / L::kPieces, piece = c % L::kPieces;
      const int row = grp * 32 + jr;
      const int blk = stage * 4 + piece * 16 / L::kBlockSrc;
      v[i] = u32x4{0u, 0u, 0u, 0u};
      if (row < rows && blk < kblocks)
        v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            src + (int64_t)row * ld_bytes + (int64_t)stage * 4 * L::kBlockSrc + piece * 16));
    }
  };
  u32x4 v[L::kCopies];
  load(work, v);
  for (;;) {
    const int grp = work / stages, stage = work - grp * stages;
    const int chunk = stage * groups + grp;
#pragma unroll
    for (int i = 0; i < L::kCopies; ++i) {
      const int c = 64 * i + lane;
      const int jr = c / L::kPieces, piece = c % L::kPieces;
      *reinterpret_cast<u32x4*>(in + jr * L::kRow + piece * 16) = v[i];
    }
    const int next = work + nwaves;
    if (next < nchunks) load(next, v);  // in flight while this chunk is converted
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    const int row = grp * 32 + j;
    uint32_t q[2][kBits];
    uint32_t sb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int qb = 2 * h + t;
      const uint8_t* p = in + j * L::kRow + qb * L::kBlockSrc;
      u32x4 w[F32 ? 8 : 4];
#pragma unroll
      for (int i = 0; i < (F32 ? 8 : 4); ++i) w[i] = *reinterpret_cast<const u32x4*>(p + 16 * i);
      sb[t] = quantize_block<FMT, F32>(w, q[t]);
      if (row >= rows || stage * 4 + qb >= kblocks) {  // padding
#pragma unroll
        for (int i = 0; i < kBits; ++i) q[t][i] = 0u;
        sb[t] = 127u;
      }
    }
    // every lane has read its blocks: the next chunk may overwrite the wave's LDS rows
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // the code bytes of row j in the planes of half h
    uint8_t* half = codes + (int64_t)chunk * chunk_codes(kBits) + h * half_codes(kBits);
    if constexpr (kBits == 6) {
      *reinterpret_cast<u32x4*>(half + kPlaneA + j * 16) = u32x4{q[0][0], q[0][1], q[0][2], q[0][3]};
      *reinterpret_cast<u32x2*>(half + kPlaneL + j * 8) = u32x2{q[0][4], q[0][5]};
      *reinterpret_cast<u32x2*>(half + kPlaneH + j * 8) = u32x2{q[1][0], q[1][1]};
      *reinterpret_cast<u32x4*>(half + kPlaneB + j * 16) = u32x4{q[1][2], q[1][3], q[1][4], q[1][5]};
    } else if constexpr (kBits == 4) {
      // 16-byte planes: block 2h, then block 2h+1
#pragma unroll
      for (int t = 0; t < 2; ++t)
        *reinterpret_cast<u32x4*>(half + t * kPlaneStride16 + j * 16) = u32x4{q[t][0], q[t][1], q[t][2], q[t][3]};
    } else {
      // 8 bits: block q = 2h + t goes to plane 2t + h of both halves, its bytes
      // 0..15 in half 0 and 16..31 in half 1
      uint8_t* chunk_base = codes + (int64_t)chunk * chunk_codes(kBits);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          *reinterpret_cast<u32x4*>(chunk_base + hh * half_codes(kBits) + (2 * t + h) * kPlaneStride16 + j * 16) =
              u32x4{q[t][4 * hh], q[t][4 * hh + 1], q[t][4 * hh + 2], q[t][4 * hh + 3]};
    }
    *reinterpret_cast<uint16_t*>(scales + (int64_t)chunk * kChunkScales + j * 4 + 2 * h) =
        (uint16_t)(sb[0] | (sb[1] << 8));
    if (next >= nchunks) break;
    work = next;
  }
}

template <int FMT>
void launch_rows_fmt(const uint8_t* s, bool f32, int64_t ldb, int64_t kblocks, int64_t total, uint8_t* codes,
                     uint8_t* scales, int vec_out, dim3 g, dim3 blk, hipStream_t stream) {
  if (f32)
    hipLaunchKernelGGL((quantize_kernel<FMT, true>), g, blk, 0, stream, s, ldb, kblocks, total, codes, scales, vec_out);
  else
    hipLaunchKernelGGL((quantize_kernel<FMT, false>), g, blk, 0, stream, s, ldb, kblocks, total, codes, scales,
                       vec_out);
}

template <int FMT>
void launch_tiled_fmt(const uint8_t* s, bool f32, int64_t ldb, int rows, int k, int groups, int nchunks,
                      uint8_t* codes, uint8_t* scales, dim3 g, dim3 blk, hipStream_t stream) {
  if (f32)
    hipLaunchKernelGGL((quantize_tiled_kernel<FMT, true>), g, blk, 0, stream, s, ldb, rows, k, groups, nchunks, codes,
                       scales);
  else
    hipLaunchKernelGGL((quantize_tiled_kernel<FMT, false>), g, blk, 0, stream, s, ldb, rows, k, groups, nchunks, codes,
                       scales);
}

}  // namespace

// rows layout: one lane per block; tiled layout: the resident workgroups walk the chunks
int64_t quantize_grid_items(int64_t rows, int64_t k, int layout) {
  if (layout == kLayoutTiled)
    return std::min<int64_t>(ceil_div(ceil_div(rows, kTileGroupRows) * ceil_div(k, kTileStageK), kTWaves),
                             kTResident) * kTWaves * 64;
  return ceil_div(rows * (k / 32), kQThreads) * kQThreads;
}

hipError_t launch_quantize(const void* src, int src_type, int64_t rows, int64_t k, int64_t ld_src, int fmt,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t kblocks = k / 32;
  const int64_t total = rows * kblocks;
  if (total == 0) return hipSuccess;
  if (quantize_grid_items(rows, k, kLayoutRows) > kMaxGridItems) return hipErrorInvalidConfiguration;
  const int64_t grid = quantize_grid_items(rows, k, kLayoutRows) / kQThreads;
  const uint8_t* s = static_cast<const uint8_t*>(src);
  const int vec_out = ((uintptr_t)codes % 16) == 0;
  const int64_t ldb = ld_src * (src_type == kSrcBf16 ? 2 : 4);
  const bool f32 = src_type == kSrcF32;
  const dim3 g((unsigned)grid), blk(kQThreads);
  switch (fmt) {
    case kFmtE2M3: launch_rows_fmt<kFmtE2M3>(s, f32, ldb, kblocks, total, codes, scales, vec_out, g, blk, stream); break;
    case kFmtE3M2: launch_rows_fmt<kFmtE3M2>(s, f32, ldb, kblocks, total, codes, scales, vec_out, g, blk, stream); break;
    case kFmtE2M1: launch_rows_fmt<kFmtE2M1>(s, f32, ldb, kblocks, total, codes, scales, vec_out, g, blk, stream); break;
    case kFmtE4M3: launch_rows_fmt<kFmtE4M3>(s, f32, ldb, kblocks, total, codes, scales, vec_out, g, blk, stream); break;
    case kFmtE5M2: launch_rows_fmt<kFmtE5M2>(s, f32, ldb, kblocks, total, codes, scales, vec_out, g, blk, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_tiled(const void* src, int src_type, int64_t rows, int64_t k, int64_t ld_src, int fmt,
                                 uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t groups = ceil_div(rows, kTileGroupRows), stages = ceil_div(k, kTileStageK);
  const int64_t nchunks = groups * stages;
  if (nchunks == 0) return hipSuccess;
  const dim3 g((unsigned)(quantize_grid_items(rows, k, kLayoutTiled) / (kTWaves * 64))), blk(kTWaves * 64);
  const uint8_t* s = static_cast<const uint8_t*>(src);
  const int64_t ldb = ld_src * (src_type == kSrcBf16 ? 2 : 4);
  const bool f32 = src_type == kSrcF32;
  const int r = (int)rows, kk = (int)k, gr = (int)groups, nc = (int)nchunks;
  switch (fmt) {
    case kFmtE2M3: launch_tiled_fmt<kFmtE2M3>(s, f32, ldb, r, kk, gr, nc, codes, scales, g, blk, stream); break;
    case kFmtE3M2: launch_tiled_fmt<kFmtE3M2>(s, f32, ldb, r, kk, gr, nc, codes, scales, g, blk, stream); break;
    case kFmtE2M1: launch_tiled_fmt<kFmtE2M1>(s, f32, ldb, r, kk, gr, nc, codes, scales, g, blk, stream); break;
    case kFmtE4M3: launch_tiled_fmt<kFmtE4M3>(s, f32, ldb, r, kk, gr, nc, codes, scales, g, blk, stream); break;
    case kFmtE5M2: launch_tiled_fmt<kFmtE5M2>(s, f32, ldb, r, kk, gr, nc, codes, scales, g, blk, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mxg
