// bf16 / fp32 -> MX (E2M3 or E3M2) quantizer for gfx950.
//
// One thread per 32-element block.  The block is read with 128-bit loads (the
// coalesced-vector-load technique of the "Creating Custom Kernels for the AMD
// MI300" page, section "Fused RMS Norm Kernel"), its amax is taken on the raw
// magnitude bits, the E8M0 scale follows the MX rule, and one v_cvt_scalef32
// instruction rounds all 32 elements.  Output: 24 bytes of packed codes and
// one scale byte per block.  HBM-bound: 2 (or 4) bytes in, 0.78 bytes out per
// element.
#include "internal.h"
#include "mx_device.h"

namespace mxg {

template <int FMT>
__global__ __launch_bounds__(256) void quantize_bf16_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                                            int64_t kblocks, int64_t total_blocks,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= total_blocks) return;
  const int64_t row = b / kblocks;
  const int64_t kb = b - row * kblocks;
  const u32x4* p = reinterpret_cast<const u32x4*>(src + row * ld_src + kb * 32);
  u32x4 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = __builtin_nontemporal_load(p + i);
  // amax on magnitude bits: for non-negative floats the bit order is the value order
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
  const BlockScale s = scale_from_bf16_bits<FMT>(amax);
  v6u q;
  if (!s.nonfinite) {
    v32bf x;
    __builtin_memcpy(&x, w, 64);
    q = cvt_bf16x32<FMT>(x, s.scale);
  } else {
    q = v6u{0, 0, 0, 0, 0, 0};
  }
  u32x2* o = reinterpret_cast<u32x2*>(codes + row * (kblocks * 24) + kb * 24);
  o[0] = u32x2{q[0], q[1]};
  o[1] = u32x2{q[2], q[3]};
  o[2] = u32x2{q[4], q[5]};
  scales[row * kblocks + kb] = (uint8_t)s.byte;
}

template <int FMT>
__global__ __launch_bounds__(256) void quantize_f32_kernel(const float* __restrict__ src, int64_t ld_src,
                                                           int64_t kblocks, int64_t total_blocks,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= total_blocks) return;
  const int64_t row = b / kblocks;
  const int64_t kb = b - row * kblocks;
  const u32x4* p = reinterpret_cast<const u32x4*>(src + row * ld_src + kb * 32);
  u32x4 w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = __builtin_nontemporal_load(p + i);
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = w[i][j] & 0x7fffffffu;
      amax = a > amax ? a : amax;
    }
  const BlockScale s = scale_from_f32_bits<FMT>(amax);
  v6u q;
  if (!s.nonfinite) {
    // element 2i of the convert comes from the first operand, 2i+1 from the second
    v16f even, odd;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      even[i] = __uint_as_float(w[i / 2][(2 * i) % 4]);
      odd[i] = __uint_as_float(w[i / 2][(2 * i) % 4 + 1]);
    }
    q = cvt_f32x2x16<FMT>(even, odd, s.scale);
  } else {
    q = v6u{0, 0, 0, 0, 0, 0};
  }
  u32x2* o = reinterpret_cast<u32x2*>(codes + row * (kblocks * 24) + kb * 24);
  o[0] = u32x2{q[0], q[1]};
  o[1] = u32x2{q[2], q[3]};
  o[2] = u32x2{q[4], q[5]};
  scales[row * kblocks + kb] = (uint8_t)s.byte;
}

hipError_t launch_quantize(const void* src, int src_type, int64_t rows, int64_t k, int64_t ld_src, int fmt,
                           uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t kblocks = k / 32;
  const int64_t total = rows * kblocks;
  if (total == 0) return hipSuccess;
  const int64_t grid = (total + 255) / 256;
  if (src_type == kSrcBf16) {
    const uint16_t* s = static_cast<const uint16_t*>(src);
    if (fmt == kFmtE2M3)
      hipLaunchKernelGGL(quantize_bf16_kernel<kFmtE2M3>, dim3((unsigned)grid), dim3(256), 0, stream, s, ld_src,
                         kblocks, total, codes, scales);
    else
      hipLaunchKernelGGL(quantize_bf16_kernel<kFmtE3M2>, dim3((unsigned)grid), dim3(256), 0, stream, s, ld_src,
                         kblocks, total, codes, scales);
  } else {
    const float* s = static_cast<const float*>(src);
    if (fmt == kFmtE2M3)
      hipLaunchKernelGGL(quantize_f32_kernel<kFmtE2M3>, dim3((unsigned)grid), dim3(256), 0, stream, s, ld_src,
                         kblocks, total, codes, scales);
    else
      hipLaunchKernelGGL(quantize_f32_kernel<kFmtE3M2>, dim3((unsigned)grid), dim3(256), 0, stream, s, ld_src,
                         kblocks, total, codes, scales);
  }
  return hipGetLastError();
}

}  // namespace mxg
