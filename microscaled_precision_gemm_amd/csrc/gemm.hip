// MX block-scaled GEMM for gfx950: C[M, N] = A[M, K] * W[N, K]^T.
//
// Design (the Krea 3 / MI355X post's kernel, section "We built a faster MXFP6
// kernel", keeps the 6-bit values packed and avoids neighbouring workgroups
// re-reading the same data; this is a new gfx950 design with those two goals):
//
//  * Operands stay packed (24 bytes per 32-element block) from HBM to the
//    matrix cores.  Each workgroup computes a 256 x 256 tile of C with 4 waves
//    of 128 x 128; K is staged 128 elements at a time through a double-buffered
//    LDS (rows padded from 96 to 112 bytes so that 16-byte reads of 8
//    consecutive rows hit distinct banks).
//  * The contraction runs on V_MFMA_SCALE_F32_32X32X64_F8F6F4: per lane 32
//    K-contiguous FP6 codes (6 VGPRs) and one E8M0 byte selected by op_sel.
//    Within a 128-element stage, lane half h of sub-step s handles K-block
//    2h + s (the K order inside one accumulation is free as long as both
//    operands agree), so every lane reads 48 contiguous bytes and its two
//    scale bytes with one 16-bit LDS read, and op_sel = s picks the byte.
//  * W is the MFMA A operand (output rows = features n) and the activations
//    the B operand (output columns = tokens m), so each lane's 16 accumulator
//    values belong to one token.  The W rows fed to the A operand are permuted
//    so that a lane holds 16 consecutive features (bf16 / fp32 output: 32- or
//    64-byte row stores), or, for the MX output, the even and odd features of
//    a half-block in the order the v_cvt_scalef32_2xpk16 instruction packs
//    them (then a lane writes 12 contiguous code bytes).
//  * Workgroups are dispatched round-robin over the 8 XCDs; tile ids are
//    remapped so that each XCD works on a contiguous range of a grouped
//    (4 m-tiles wide) tile order and the tiles in flight on one XCD share A
//    and W slices in that XCD's L2.
#include "internal.h"
#include "mx_device.h"

namespace mxg {

namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 96;   // 128 FP6 codes
constexpr int kLdsRow = 112;    // padded LDS row stride
constexpr int kTileBytes = kTileM * kLdsRow;
constexpr int kOffX = 0;
constexpr int kOffW = kTileBytes;
constexpr int kOffXs = 2 * kTileBytes;
constexpr int kOffWs = 2 * kTileBytes + kTileM * 4;
constexpr int kStageBytes = 2 * kTileBytes + 2 * kTileM * 4;
constexpr int kLdsBytes = 2 * kStageBytes;
static_assert(kTileM == kTileN, "the loader assumes square tiles");
static_assert(kLdsBytes <= 160 * 1024, "gfx950 LDS is 160 KB per workgroup");

constexpr int kLayoutContig = 0;  // lane holds features 16h .. 16h+15 of a 32-feature fragment
constexpr int kLayoutMx = 1;      // lane holds features 16h + {0,2,..,14} then 16h + {1,3,..,15}

// Feature (n) offset inside a 32-row fragment for MFMA A-operand row j.  The
// 32x32 output has lane l, register r at row 8(r/4) + 4(l/32) + r%4, column l%32.
template <int LAYOUT>
__device__ __forceinline__ int feature_of_row(int j) {
  const int a = j >> 3, h = (j >> 2) & 1, b = j & 3;
  const int r = 4 * a + b;
  if constexpr (LAYOUT == kLayoutContig)
    return 16 * h + r;
  else
    return 16 * h + (r < 8 ? 2 * r : 2 * (r - 8) + 1);
}

// XCD-aware tile order: contiguous ranges per XCD, grouped 4 m-tiles wide.
__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int s = b;
  if (total >= 64) {
    const int xcd = b & 7, idx = b >> 3;
    const int per = total >> 3, rem = total & 7;
    s = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  }
  constexpr int kGroupM = 4;
  const int group = s / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in = s - group * kGroupM * tiles_n;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &a, 2);
  __builtin_memcpy(&ub, &b, 2);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

template <int WF, int XF, int S>
__device__ __forceinline__ void mfma_substep(v16f (&acc)[4][4], const u32x4 (&wd)[4][3], const u32x4 (&xd)[4][3],
                                             const uint32_t (&wsc)[4], const uint32_t (&xsc)[4]) {
  v8i a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    if constexpr (S == 0) {
      a[f] = v8i{(int)wd[f][0][0], (int)wd[f][0][1], (int)wd[f][0][2], (int)wd[f][0][3],
                 (int)wd[f][1][0], (int)wd[f][1][1], 0, 0};
      b[f] = v8i{(int)xd[f][0][0], (int)xd[f][0][1], (int)xd[f][0][2], (int)xd[f][0][3],
                 (int)xd[f][1][0], (int)xd[f][1][1], 0, 0};
    } else {
      a[f] = v8i{(int)wd[f][1][2], (int)wd[f][1][3], (int)wd[f][2][0], (int)wd[f][2][1],
                 (int)wd[f][2][2], (int)wd[f][2][3], 0, 0};
      b[f] = v8i{(int)xd[f][1][2], (int)xd[f][1][3], (int)xd[f][2][0], (int)xd[f][2][1],
                 (int)xd[f][2][2], (int)xd[f][2][3], 0, 0};
    }
  }
#pragma unroll
  for (int fn = 0; fn < 4; ++fn)
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
      acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[fn], b[fm], acc[fn][fm], WF, XF, S,
                                                                    (int)wsc[fn], S, (int)xsc[fm]);
}

template <int WF, int XF, int OUT, bool GELU, int OFMT>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  constexpr int kLayout = OUT == kOutMx ? kLayoutMx : kLayoutContig;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int tm, tn;
  tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * kTileM, n0 = tn * kTileN;
  const int64_t rowbytes = (int64_t)g.K * 3 / 4;
  const int kblocks = g.K / 32;
  const int nk = (g.K + kStageK - 1) / kStageK;
  const bool kaligned = (g.K % kStageK) == 0;

  // ---- global -> register loader: 6 chunks of 16 bytes per operand per thread
  const uint8_t* xsrc[6];
  const uint8_t* wsrc[6];
  int lds_off[6], part16[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int c = tid + kThreads * i;
    const int row = c / 6, part = c - 6 * row;
    const int xr = min(m0 + row, g.M - 1), wr = min(n0 + row, g.N - 1);
    xsrc[i] = g.x_codes + (int64_t)xr * rowbytes + part * 16;
    wsrc[i] = g.w_codes + (int64_t)wr * rowbytes + part * 16;
    lds_off[i] = row * kLdsRow + part * 16;
    part16[i] = part * 16;
  }
  const uint8_t* xs_src = g.x_scales + (int64_t)min(m0 + tid, g.M - 1) * kblocks;
  const uint8_t* ws_src = g.w_scales + (int64_t)min(n0 + tid, g.N - 1) * kblocks;

  u32x4 xreg[6], wreg[6];
  uint32_t xsreg = 0, wsreg = 0;

  auto gload = [&](int ks) {
    const int64_t koff = (int64_t)ks * kRowBytes;
    if (kaligned || ks < nk - 1) {
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        xreg[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + koff);
        wreg[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + koff);
      }
    } else {
      // last, partial stage: valid bytes per row are a multiple of 24 (whole blocks)
      const int valid = (int)(rowbytes - koff);
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        if (part16[i] + 16 <= valid) {
          xreg[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + koff);
          wreg[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + koff);
        } else if (part16[i] + 8 <= valid) {
          const u32x2 xh = *reinterpret_cast<const u32x2*>(xsrc[i] + koff);
          const u32x2 wh = *reinterpret_cast<const u32x2*>(wsrc[i] + koff);
          xreg[i] = u32x4{xh[0], xh[1], 0u, 0u};
          wreg[i] = u32x4{wh[0], wh[1], 0u, 0u};
        } else {
          xreg[i] = u32x4{0u, 0u, 0u, 0u};
          wreg[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    if (kaligned) {
      xsreg = *reinterpret_cast<const uint32_t*>(xs_src + 4 * ks);
      wsreg = *reinterpret_cast<const uint32_t*>(ws_src + 4 * ks);
    } else {
      // scale rows are not 4-byte aligned; blocks past K get 2^0 (their codes are 0)
      uint32_t xv = 0, wv = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int blk = 4 * ks + b;
        const uint32_t xb = blk < kblocks ? xs_src[blk] : 127u;
        const uint32_t wb = blk < kblocks ? ws_src[blk] : 127u;
        xv |= xb << (8 * b);
        wv |= wb << (8 * b);
      }
      xsreg = xv;
      wsreg = wv;
    }
  };
  auto lstore = [&](int buf) {
    uint8_t* st = lds + buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      *reinterpret_cast<u32x4*>(st + kOffX + lds_off[i]) = xreg[i];
      *reinterpret_cast<u32x4*>(st + kOffW + lds_off[i]) = wreg[i];
    }
    *reinterpret_cast<uint32_t*>(st + kOffXs + tid * 4) = xsreg;
    *reinterpret_cast<uint32_t*>(st + kOffWs + tid * 4) = wsreg;
  };

  // ---- per-lane LDS read offsets for the MFMA operands
  const int wn = wave & 1, wm = wave >> 1;
  const int h = lane >> 5, j = lane & 31;
  const int wrow = feature_of_row<kLayout>(j);
  int w_off[4], x_off[4], ws_off[4], xs_off[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int wr = wn * 128 + f * 32 + wrow;
    const int xr = wm * 128 + f * 32 + j;
    w_off[f] = kOffW + wr * kLdsRow + 48 * h;
    x_off[f] = kOffX + xr * kLdsRow + 48 * h;
    ws_off[f] = kOffWs + wr * 4 + 2 * h;
    xs_off[f] = kOffXs + xr * 4 + 2 * h;
  }

  v16f acc[4][4];
#pragma unroll
  for (int fn = 0; fn < 4; ++fn)
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fn][fm][r] = 0.0f;

  auto compute = [&](int buf) {
    const uint8_t* st = lds + buf * kStageBytes;
    u32x4 wd[4][3], xd[4][3];
    uint32_t wsc[4], xsc[4];
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        wd[f][q] = *reinterpret_cast<const u32x4*>(st + w_off[f] + 16 * q);
        xd[f][q] = *reinterpret_cast<const u32x4*>(st + x_off[f] + 16 * q);
      }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      wsc[f] = *reinterpret_cast<const uint16_t*>(st + ws_off[f]);
      xsc[f] = *reinterpret_cast<const uint16_t*>(st + xs_off[f]);
    }
    mfma_substep<WF, XF, 0>(acc, wd, xd, wsc, xsc);
    mfma_substep<WF, XF, 1>(acc, wd, xd, wsc, xsc);
  };

  // ---- main loop: one barrier per stage, next stage's global loads in flight during the MFMAs
  if (nk > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const bool more = ks + 1 < nk;
    if (more) gload(ks + 1);
    compute(ks & 1);
    if (more) lstore((ks + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue
  const int mw0 = m0 + wm * 128, nw0 = n0 + wn * 128;
#pragma unroll
  for (int fn = 0; fn < 4; ++fn) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
      const int m = mw0 + fm * 32 + j;
      v16f v = acc[fn][fm];
      if constexpr (GELU) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = gelu_tanh_f32(v[r]);
      }
      if constexpr (OUT == kOutMx) {
        const int nb = nw0 + fn * 32;  // first feature of this 32-wide block
        uint32_t amax = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t a = __float_as_uint(v[r]) & 0x7fffffffu;
          amax = a > amax ? a : amax;
        }
        const uint32_t other = (uint32_t)__shfl_xor((int)amax, 32);
        amax = other > amax ? other : amax;
        const BlockScale sc = scale_from_f32_bits<OFMT>(amax);
        v16f ev, od;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          ev[i] = i < 8 ? v[i] : 0.0f;
          od[i] = i < 8 ? v[8 + i] : 0.0f;
        }
        v6u q = cvt_f32x2x16<OFMT>(ev, od, sc.scale);
        if (sc.nonfinite) q = v6u{0, 0, 0, 0, 0, 0};
        if (m < g.M && nb < g.N) {
          uint8_t* codes = static_cast<uint8_t*>(g.out);
          uint32_t* o = reinterpret_cast<uint32_t*>(codes + (int64_t)m * (g.N / 32 * 24) + (nb / 32) * 24 + 12 * h);
          o[0] = q[0];
          o[1] = q[1];
          o[2] = q[2];
          if (h == 0) g.out_scales[(int64_t)m * (g.N / 32) + nb / 32] = (uint8_t)sc.byte;
        }
      } else {
        const int n = nw0 + fn * 32 + 16 * h;
        if (m < g.M) {
          if constexpr (OUT == kOutBf16) {
            uint16_t* out = static_cast<uint16_t*>(g.out) + (int64_t)m * g.ldo;
            if (g.vec_store && n + 16 <= g.N) {
              u32x4* o = reinterpret_cast<u32x4*>(out + n);
              o[0] = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                           pack_bf16x2(v[6], v[7])};
              o[1] = u32x4{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
                           pack_bf16x2(v[14], v[15])};
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (n + r < g.N) {
                  const __bf16 b = (__bf16)v[r];
                  __builtin_memcpy(out + n + r, &b, 2);
                }
            }
          } else {
            float* out = static_cast<float*>(g.out) + (int64_t)m * g.ldo;
            if (g.vec_store && n + 16 <= g.N) {
              u32x4* o = reinterpret_cast<u32x4*>(out + n);
#pragma unroll
              for (int q = 0; q < 4; ++q)
                o[q] = u32x4{__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                             __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3])};
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (n + r < g.N) out[n + r] = v[r];
            }
          }
        }
      }
    }
  }
}

template <int WF, int XF>
hipError_t launch_formats(const GemmArgs& a, int epilogue, int out_kind, int out_fmt, hipStream_t stream) {
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(kThreads);
  const bool gelu = epilogue == kEpiGeluTanh;
  if (out_kind == kOutF32) {
    if (gelu)
      hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutF32, true, kFmtE2M3>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutF32, false, kFmtE2M3>), grid, block, 0, stream, a);
  } else if (out_kind == kOutBf16) {
    if (gelu)
      hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutBf16, true, kFmtE2M3>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutBf16, false, kFmtE2M3>), grid, block, 0, stream, a);
  } else {
    if (out_fmt == kFmtE2M3) {
      if (gelu)
        hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutMx, true, kFmtE2M3>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutMx, false, kFmtE2M3>), grid, block, 0, stream, a);
    } else {
      if (gelu)
        hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutMx, true, kFmtE3M2>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutMx, false, kFmtE3M2>), grid, block, 0, stream, a);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, int x_fmt, int w_fmt, int epilogue, int out_kind, int out_fmt,
                       hipStream_t stream) {
  if (w_fmt == kFmtE2M3 && x_fmt == kFmtE2M3) return launch_formats<kFmtE2M3, kFmtE2M3>(a, epilogue, out_kind, out_fmt, stream);
  if (w_fmt == kFmtE3M2 && x_fmt == kFmtE2M3) return launch_formats<kFmtE3M2, kFmtE2M3>(a, epilogue, out_kind, out_fmt, stream);
  if (w_fmt == kFmtE2M3 && x_fmt == kFmtE3M2) return launch_formats<kFmtE2M3, kFmtE3M2>(a, epilogue, out_kind, out_fmt, stream);
  return hipErrorInvalidValue;  // E3M2 x E3M2 is rejected by the front end
}

}  // namespace mxg
