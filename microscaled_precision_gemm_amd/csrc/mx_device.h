// Device-side helpers shared by the gfx950 kernels: vector types, the MX scale
// rule on raw float bits, and the hardware FP6 conversions.
//
// The MX rule (OCP Microscaling v1.0, the format the Krea 3 / MI355X post uses
// for its MLPs, section "Quality set the precision limit"): for a block of 32
// values, shared = clamp(floor(log2 amax) - emax_elem, -127, 127), scale byte =
// shared + 127, elements = RNE(v / 2^shared) saturated.  floor(log2 amax) is
// read exactly from the exponent bits (leading-one position for subnormals).
// The element rounding is done by gfx950's v_cvt_scalef32_* instructions,
// which divide by the fp32 scale operand and round to nearest even with
// saturation and a kept sign bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace mxg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v6u __attribute__((ext_vector_type(6)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v32bf __attribute__((ext_vector_type(32)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

typedef short v2s __attribute__((ext_vector_type(2)));

// floor(log2(max magnitude)) of the element format: E2M3 7.5 = 1.875 * 2^2,
// E3M2 28 = 1.75 * 2^4, E2M1 6 = 1.5 * 2^2, E4M3 448 = 1.75 * 2^8, E5M2
// 57344 = 1.75 * 2^15.
template <int FMT>
__device__ __forceinline__ constexpr int emax_elem() {
  return FMT == kFmtE2M3 ? 2 : FMT == kFmtE3M2 ? 4 : FMT == kFmtE2M1 ? 2 : FMT == kFmtE4M3 ? 8 : 15;
}

// Largest finite magnitude of the element format.
template <int FMT>
__device__ __forceinline__ constexpr float max_elem() {
  return FMT == kFmtE2M3 ? 7.5f : FMT == kFmtE3M2 ? 28.0f : FMT == kFmtE2M1 ? 6.0f : FMT == kFmtE4M3 ? 448.0f : 57344.0f;
}

// Result of the scale rule for one block.
struct BlockScale {
  float scale;     // 2^shared as an fp32 operand for the convert (2^-127 is the subnormal 0x00400000)
  uint32_t byte;   // E8M0 byte; 0xFF marks a non-finite block
  bool nonfinite;
};

// shared exponent -> (E8M0 byte, fp32 scale operand), shared already clamped to [-127, 127].
__device__ __forceinline__ BlockScale make_scale(int shared) {
  BlockScale s;
  s.byte = (uint32_t)(shared + 127);
  s.scale = shared >= -126 ? __uint_as_float((uint32_t)(shared + 127) << 23) : __uint_as_float(0x00400000u);
  s.nonfinite = false;
  return s;
}

// Scale rule from the magnitude bits of an fp32 amax (sign bit clear).
template <int FMT>
__device__ __forceinline__ BlockScale scale_from_f32_bits(uint32_t amax_bits) {
  if (amax_bits >= 0x7f800000u) {
    BlockScale s;
    s.byte = 0xFFu;
    s.scale = 1.0f;
    s.nonfinite = true;
    return s;
  }
  int fl;
  const uint32_t e = amax_bits >> 23;
  if (e != 0) {
    fl = (int)e - 127;
  } else {
    const uint32_t m = amax_bits & 0x7fffffu;
    fl = m ? (-149 + 31 - __clz((int)m)) : -100000;  // subnormal: m * 2^-149
  }
  int shared = fl - emax_elem<FMT>();
  shared = shared < -127 ? -127 : (shared > 127 ? 127 : shared);
  return make_scale(shared);
}

// Running block amax of fp32 values: max(m, |a|, |b|) in one v_maximum3_f32.
// Unlike v_max3 it propagates a NaN, so the bits of the result order exactly
// as the integer maximum of the magnitude bits would: a block holding a NaN or
// an infinity ends at bits >= 0x7f800000 (the non-finite scale), any other
// block at its largest magnitude.
__device__ __forceinline__ float absmax2(float m, float a, float b) {
  return __builtin_elementwise_maximum(m, __builtin_elementwise_maximum(__builtin_fabsf(a), __builtin_fabsf(b)));
}

// Scale rule from the magnitude bits of a bf16 amax (sign bit clear, in the low 16 bits).
template <int FMT>
__device__ __forceinline__ BlockScale scale_from_bf16_bits(uint32_t amax_bits) {
  return scale_from_f32_bits<FMT>(amax_bits << 16);
}

// The scaled FP6 conversions below are written as inline asm with an
// early-clobber result.  They produce their 6 result dwords over several
// passes and read the scale operand again after the first one: if the
// destination tuple starts on the scale's register, every element after the
// first pass is converted with a clobbered scale.  The compiler's register
// allocator does not know this and can assign such an overlap, so the result
// is kept apart from all inputs.

// 32 bf16 values -> 32 FP6 codes packed as 6 dwords (element i at bits [6i, 6i+6)).
template <int FMT>
__device__ __forceinline__ v6u cvt_bf16x32(v32bf x, float scale) {
  v6u r;
  if constexpr (FMT == kFmtE2M3)
    asm("v_cvt_scalef32_pk32_fp6_bf16 %0, %1, %2" : "=&v"(r) : "v"(x), "v"(scale));
  else
    asm("v_cvt_scalef32_pk32_bf6_bf16 %0, %1, %2" : "=&v"(r) : "v"(x), "v"(scale));
  return r;
}

// Two 16-float vectors -> 32 FP6 codes; output element 2i comes from a[i] and
// element 2i+1 from b[i] (the instruction interleaves its two sources).
template <int FMT>
__device__ __forceinline__ v6u cvt_f32x2x16(v16f a, v16f b, float scale) {
  v6u r;
  if constexpr (FMT == kFmtE2M3)
    asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(r) : "v"(a), "v"(b), "v"(scale));
  else
    asm("v_cvt_scalef32_2xpk16_bf6_f32 %0, %1, %2, %3" : "=&v"(r) : "v"(a), "v"(b), "v"(scale));
  return r;
}

// One block of 32 fp32 values (element i in v[i]) -> its codes packed as
// fmt_bits(FMT) dwords (element i at bits [b*i, b*i+b) of the block; E2M1:
// element 2i in the low nibble of byte i).  The 6-bit types go through the
// 2 x 16 conversion above, which saturates by itself.  For the 8- and 4-bit
// types the values are first clamped to +-max_elem * scale (exact in fp32, an
// infinity only where no finite input can exceed it), so the conversion only
// rounds: its handling of out-of-range inputs never enters.  The clamp keeps
// the sign of zeros.
template <int FMT>
__device__ __forceinline__ void cvt_block(const float (&v)[32], float scale, uint32_t (&q)[fmt_bits(FMT)]) {
  if constexpr (fmt_bits(FMT) == 6) {
    v16f even, odd;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      even[i] = v[2 * i];
      odd[i] = v[2 * i + 1];
    }
    const v6u r = cvt_f32x2x16<FMT>(even, odd, scale);
#pragma unroll
    for (int i = 0; i < 6; ++i) q[i] = r[i];
  } else {
    const float bound = max_elem<FMT>() * scale;
    auto cl = [&](float x) { return __builtin_amdgcn_fmed3f(x, -bound, bound); };
    if constexpr (fmt_bits(FMT) == 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v2s w = {0, 0};
        if constexpr (FMT == kFmtE4M3) {
          w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, cl(v[4 * i]), cl(v[4 * i + 1]), scale, false);
          w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, cl(v[4 * i + 2]), cl(v[4 * i + 3]), scale, true);
        } else {
          w = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(w, cl(v[4 * i]), cl(v[4 * i + 1]), scale, false);
          w = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(w, cl(v[4 * i + 2]), cl(v[4 * i + 3]), scale, true);
        }
        __builtin_memcpy(&q[i], &w, 4);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, cl(v[8 * i]), cl(v[8 * i + 1]), scale, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, cl(v[8 * i + 2]), cl(v[8 * i + 3]), scale, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, cl(v[8 * i + 4]), cl(v[8 * i + 5]), scale, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, cl(v[8 * i + 6]), cl(v[8 * i + 7]), scale, 3);
        q[i] = w;
      }
    }
  }
}

// GELU, tanh form, in fp32: 0.5 x (1 + tanh(u)) = x / (1 + e^{-2u}) with
// u = sqrt(2/pi) (x + 0.044715 x^3) (Hendrycks & Gimpel).  e^{-2u} is taken as
// 2^{-2u log2 e} with the hardware exp2 and the quotient with the hardware
// reciprocal; for very negative x, 2^{...} overflows to +inf and the result is
// x * 0 = -0.
__device__ __forceinline__ float gelu_tanh_f32(float x) {
  // -2u log2 e = x (c0 + c1 x^2) with c0 = -2 sqrt(2/pi) log2 e, c1 = 0.044715 c0
  constexpr float kC0 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
  constexpr float kC1 = kC0 * 0.044715f;
  const float t = __builtin_amdgcn_exp2f(x * __builtin_fmaf(kC1, x * x, kC0));
  return x * __builtin_amdgcn_rcpf(1.0f + t);
}

// SiLU in fp32: x * sigmoid(x) = x / (1 + e^{-x}), with e^{-x} taken as
// 2^{-x log2 e} by the hardware exp2 and the quotient by the hardware
// reciprocal; for very negative x the power overflows to +inf and the result
// is x * 0 = -0.
__device__ __forceinline__ float silu_f32(float x) {
  constexpr float kNegLog2e = -1.4426950408889634f;
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * kNegLog2e));
}

}  // namespace mxg
