// bf16 / fp32 -> MX (E2M3 or E3M2) quantizer for gfx950.
//
// Each wave quantizes 64 consecutive 32-element blocks (row-major order over
// [rows, K/32]).  HBM-bound (2 or 4 bytes in, 0.78 bytes out per element), so
// the design is about full-width memory transactions:
//
//  * loads: the wave reads its blocks as 16-byte pieces with consecutive lanes
//    on consecutive pieces (the 128-bit coalesced loads of the page "Creating
//    Custom Kernels for the AMD MI300", section "Fused RMS Norm Kernel"), and
//    an LDS transpose hands each lane one whole block;
//  * per block: amax on the raw magnitude bits, the E8M0 scale from the
//    exponent bits, and one v_cvt_scalef32 instruction that rounds all 32
//    elements (round-to-nearest-even, saturating, sign kept);
//  * stores: the 64 x 24 code bytes of a wave are contiguous in the output, so
//    they go back through LDS and leave as 16-byte stores of consecutive lanes.
#include "internal.h"
#include "mx_device.h"

namespace mxg {

namespace {

constexpr int kQThreads = 256;
constexpr int kQWaves = kQThreads / 64;
constexpr int kInRowB = 16 * 5;                  // one block's bf16 bytes (64) padded to 80 for the LDS read
constexpr int kInRowF = 16 * 9;                  // fp32 (128) padded to 144
constexpr int kOutBytes = 64 * 24;               // code bytes of one wave

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
  const int64_t b = wave_first + lane;
  u32x4 w[L::kPieces];
#pragma unroll
  for (int i = 0; i < L::kPieces; ++i) w[i] = *reinterpret_cast<const u32x4*>(in + lane * L::kRow + i * 16);
  BlockScale s;
  v6u q;
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
    const uint32_t amax = m2[0] > m2[1] ? m2[0] : m2[1];
    s = scale_from_bf16_bits<FMT>(amax);
    v32bf x;
    __builtin_memcpy(&x, w, 64);
    q = cvt_bf16x32<FMT>(x, s.scale);
  } else {
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t a = w[i][j] & 0x7fffffffu;
        amax = a > amax ? a : amax;
      }
    s = scale_from_f32_bits<FMT>(amax);
    // element 2i of the convert comes from the first operand, 2i+1 from the second
    v16f even, odd;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      even[i] = __uint_as_float(w[i / 2][(2 * i) % 4]);
      odd[i] = __uint_as_float(w[i / 2][(2 * i) % 4 + 1]);
    }
    q = cvt_f32x2x16<FMT>(even, odd, s.scale);
  }
  if (s.nonfinite) q = v6u{0, 0, 0, 0, 0, 0};
  if (b < total_blocks) scales[b] = (uint8_t)s.byte;

  // ---- stores: the wave's code bytes are contiguous at codes + 24 * wave_first
  const int nblk = (int)min((int64_t)64, total_blocks - wave_first);
  if (vec_out && nblk == 64) {
    u32x2* o = reinterpret_cast<u32x2*>(outb + 24 * lane);
    o[0] = u32x2{q[0], q[1]};
    o[1] = u32x2{q[2], q[3]};
    o[2] = u32x2{q[4], q[5]};
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    uint8_t* dst = codes + 24 * wave_first;
    *reinterpret_cast<u32x4*>(dst + 16 * lane) = *reinterpret_cast<const u32x4*>(outb + 16 * lane);
    if (lane < 32)
      *reinterpret_cast<u32x4*>(dst + 1024 + 16 * lane) = *reinterpret_cast<const u32x4*>(outb + 1024 + 16 * lane);
  } else if (b < total_blocks) {
    u32x2* o = reinterpret_cast<u32x2*>(codes + 24 * b);
    o[0] = u32x2{q[0], q[1]};
    o[1] = u32x2{q[2], q[3]};
    o[2] = u32x2{q[4], q[5]};
  }
}

// ---- tiled layout: one wave per (stage, 32-row group) chunk of 32 rows x 128
// elements.  Loads: 256 (bf16) or 512 (fp32) contiguous bytes per row, 16 per
// lane, consecutive lanes on consecutive bytes.  Each lane then converts two
// blocks of one row (blocks 2h, 2h+1 for lane half h), whose 48 code bytes
// fill that row's entries of the four planes of half h: the 32 lanes of a half
// write runs of 512, 256, 256 and 512 contiguous bytes.  Rows >= rows and
// blocks >= K/32 are written as padding (codes 0, scale 127).
constexpr int kTWaves = 4;

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
  const int chunk = blockIdx.x * kTWaves + wave;
  if (chunk >= nchunks) return;  // wave-level only: no workgroup barrier below
  const int stage = chunk / groups, grp = chunk - stage * groups;
  uint8_t* in = lds + wave * 32 * L::kRow;
  const int kblocks = k / 32;

#pragma unroll
  for (int i = 0; i < L::kCopies; ++i) {
    const int c = 64 * i + lane;
    const int jr = c / L::kPieces, piece = c % L::kPieces;
    const int row = grp * 32 + jr;
    const int blk = stage * 4 + piece * 16 / L::kBlockSrc;  // block this 16-byte piece belongs to
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row < rows && blk < kblocks)
      v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          src + (int64_t)row * ld_bytes + (int64_t)stage * 4 * L::kBlockSrc + piece * 16));
    *reinterpret_cast<u32x4*>(in + jr * L::kRow + piece * 16) = v;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

  const int j = lane & 31, h = lane >> 5;
  const int row = grp * 32 + j;
  v6u q[2];
  uint32_t sb[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int qb = 2 * h + t;
    const uint8_t* p = in + j * L::kRow + qb * L::kBlockSrc;
    BlockScale s;
    v6u r;
    if constexpr (!F32) {
      u32x4 w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = *reinterpret_cast<const u32x4*>(p + 16 * i);
      u16x2 m2 = {0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a = w[i][e] & 0x7fff7fffu;
          u16x2 vv;
          __builtin_memcpy(&vv, &a, 4);
          m2 = __builtin_elementwise_max(m2, vv);
        }
      s = scale_from_bf16_bits<FMT>(m2[0] > m2[1] ? m2[0] : m2[1]);
      v32bf x;
      __builtin_memcpy(&x, w, 64);
      r = cvt_bf16x32<FMT>(x, s.scale);
    } else {
      u32x4 w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = *reinterpret_cast<const u32x4*>(p + 16 * i);
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a = w[i][e] & 0x7fffffffu;
          amax = a > amax ? a : amax;
        }
      s = scale_from_f32_bits<FMT>(amax);
      v16f even, odd;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        even[i] = __uint_as_float(w[i / 2][(2 * i) % 4]);
        odd[i] = __uint_as_float(w[i / 2][(2 * i) % 4 + 1]);
      }
      r = cvt_f32x2x16<FMT>(even, odd, s.scale);
    }
    uint32_t byte = s.byte;
    if (s.nonfinite) r = v6u{0, 0, 0, 0, 0, 0};
    if (row >= rows || stage * 4 + qb >= kblocks) {  // padding
      r = v6u{0, 0, 0, 0, 0, 0};
      byte = 127u;
    }
    q[t] = r;
    sb[t] = byte;
  }
  // the 48 code bytes of row j in the planes of half h
  uint8_t* half = codes + (int64_t)chunk * kChunkCodes + h * kHalfBytes;
  *reinterpret_cast<u32x4*>(half + kPlaneA + j * 16) = u32x4{q[0][0], q[0][1], q[0][2], q[0][3]};
  *reinterpret_cast<u32x2*>(half + kPlaneL + j * 8) = u32x2{q[0][4], q[0][5]};
  *reinterpret_cast<u32x2*>(half + kPlaneH + j * 8) = u32x2{q[1][0], q[1][1]};
  *reinterpret_cast<u32x4*>(half + kPlaneB + j * 16) = u32x4{q[1][2], q[1][3], q[1][4], q[1][5]};
  *reinterpret_cast<uint16_t*>(scales + (int64_t)chunk * kChunkScales + j * 4 + 2 * h) =
      (uint16_t)(sb[0] | (sb[1] << 8));
}

}  // namespace

hipError_t launch_quantize(const void* src, int src_type, int64_t rows, int64_t k, int64_t ld_src, int fmt,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t kblocks = k / 32;
  const int64_t total = rows * kblocks;
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + 64 * kQWaves - 1) / (64 * kQWaves);
  const uint8_t* s = static_cast<const uint8_t*>(src);
  const int vec_out = ((uintptr_t)codes % 16) == 0;
  const int64_t esize = src_type == kSrcBf16 ? 2 : 4;
  const dim3 g((unsigned)grid), blk(kQThreads);
  if (src_type == kSrcBf16) {
    if (fmt == kFmtE2M3)
      hipLaunchKernelGGL((quantize_kernel<kFmtE2M3, false>), g, blk, 0, stream, s, ld_src * esize, kblocks, total,
                         codes, scales, vec_out);
    else
      hipLaunchKernelGGL((quantize_kernel<kFmtE3M2, false>), g, blk, 0, stream, s, ld_src * esize, kblocks, total,
                         codes, scales, vec_out);
  } else {
    if (fmt == kFmtE2M3)
      hipLaunchKernelGGL((quantize_kernel<kFmtE2M3, true>), g, blk, 0, stream, s, ld_src * esize, kblocks, total,
                         codes, scales, vec_out);
    else
      hipLaunchKernelGGL((quantize_kernel<kFmtE3M2, true>), g, blk, 0, stream, s, ld_src * esize, kblocks, total,
                         codes, scales, vec_out);
  }
  return hipGetLastError();
}

}  // namespace mxg

namespace mxg {

hipError_t launch_quantize_tiled(const void* src, int src_type, int64_t rows, int64_t k, int64_t ld_src, int fmt,
                                 uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t groups = ceil_div(rows, kTileGroupRows), stages = ceil_div(k, kTileStageK);
  const int64_t nchunks = groups * stages;
  if (nchunks == 0) return hipSuccess;
  const dim3 g((unsigned)ceil_div(nchunks, kTWaves)), blk(kTWaves * 64);
  const uint8_t* s = static_cast<const uint8_t*>(src);
  const int64_t ldb = ld_src * (src_type == kSrcBf16 ? 2 : 4);
  if (src_type == kSrcBf16) {
    if (fmt == kFmtE2M3)
      hipLaunchKernelGGL((quantize_tiled_kernel<kFmtE2M3, false>), g, blk, 0, stream, s, ldb, (int)rows, (int)k,
                         (int)groups, (int)nchunks, codes, scales);
    else
      hipLaunchKernelGGL((quantize_tiled_kernel<kFmtE3M2, false>), g, blk, 0, stream, s, ldb, (int)rows, (int)k,
                         (int)groups, (int)nchunks, codes, scales);
  } else {
    if (fmt == kFmtE2M3)
      hipLaunchKernelGGL((quantize_tiled_kernel<kFmtE2M3, true>), g, blk, 0, stream, s, ldb, (int)rows, (int)k,
                         (int)groups, (int)nchunks, codes, scales);
    else
      hipLaunchKernelGGL((quantize_tiled_kernel<kFmtE3M2, true>), g, blk, 0, stream, s, ldb, (int)rows, (int)k,
                         (int)groups, (int)nchunks, codes, scales);
  }
  return hipGetLastError();
}

}  // namespace mxg
