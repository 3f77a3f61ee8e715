// MX block-scaled GEMM for gfx950: C[M, N] = A[M, K] * W[N, K]^T with both
// operands in the tiled MX layout (see include/mxgemm.h).
//
// The Krea 3 / MI355X post's kernel (section "We built a faster MXFP6
// kernel") keeps the 6-bit values packed and stops neighbouring workgroups
// from re-reading the same data; this is a new gfx950 design with those goals:
//
//  * Operands stay packed (24 bytes per 32-element block) from HBM to the
//    matrix cores.  A workgroup computes a 256 x 256 tile of C with 4 waves of
//    128 x 128 on V_MFMA_SCALE_F32_32X32X64_F8F6F4 (per lane 32 K-contiguous
//    FP6 codes in 6 VGPRs and one E8M0 byte picked by op_sel).
//  * K advances in stages of 128.  In the tiled layout one stage of 256 rows
//    is a contiguous 24 KB run, so each stage is brought in by
//    global_load_lds_dwordx4 copies straight into LDS (no VGPR staging), into
//    a ring of 3 stages: two stages are in flight while the third is
//    consumed.  The waits on those copies are explicit (s_waitcnt vmcnt) and
//    the barrier is a bare s_barrier, so a stage only waits for its own data.
//    The copies are issued one after every second MFMA of the current stage,
//    so the address path and the matrix cores work side by side.
//  * Inside a stage, lane half h of sub-step s handles K-block 2h + s (the K
//    order inside one accumulation is free as long as both operands agree):
//    each lane reads 3 consecutive 16-byte pieces (48 bytes) and a 16-bit
//    scale pair; op_sel = s picks the byte.  The tiled layout stores piece p
//    of a 32-row group contiguously, so the 32 lanes of a half read 512
//    consecutive bytes (no LDS bank conflicts from row strides).
//  * W is the MFMA A operand (output rows = features n), the activations the
//    B operand (columns = tokens m), so each lane's 16 accumulators belong to
//    one token.  The W rows fed to the A operand are permuted so that a lane
//    holds 16 consecutive features (bf16 / fp32 output: 32- or 64-byte
//    stores), or, for the MX output, the even and odd features of a
//    half-block in the order the v_cvt_scalef32_2xpk16 instruction packs them.
//  * Workgroups are dispatched round-robin over the 8 XCDs; tile ids are
//    remapped so that each XCD works on a contiguous range of a grouped
//    (4 m-tiles wide) tile order and the tiles in flight on one XCD share A
//    and W stages in that XCD's L2.
#pragma once

#include <type_traits>

#include "internal.h"
#include "mx_device.h"

namespace mxg {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;
constexpr int kRing = 3;
constexpr int kGroupsPerTile = kTileM / kTileGroupRows;            // 8
constexpr int kStageCodes = kGroupsPerTile * kChunkCodes;           // 24 KB per operand
constexpr int kStageScales = kGroupsPerTile * kChunkScales;         // 1 KB per operand
constexpr int kOffX = 0;
constexpr int kOffW = kStageCodes;
constexpr int kOffXs = 2 * kStageCodes;
constexpr int kOffWs = 2 * kStageCodes + kStageScales;
constexpr int kSlotBytes = 2 * kStageCodes + 2 * kStageScales;      // 51200
constexpr int kLdsBytes = kRing * kSlotBytes;                       // 153600
constexpr int kCodeCopiesPerWave = kStageCodes / 1024 / 4;          // 6 x 1 KB per operand
constexpr int kCopiesPerStage = 2 * kCodeCopiesPerWave + 2;         // per wave: codes + one scale copy each
static_assert(kTileM == kTileN, "the loader assumes square tiles");
static_assert(kLdsBytes <= 160 * 1024, "gfx950 LDS is 160 KB per workgroup");
static_assert(kStageScales == 4 * 64 * 4, "one 4-byte copy per lane per wave covers a stage's scales");

// s_waitcnt immediate (gfx9 encoding): vmcnt <= vm, lgkmcnt == 0, expcnt not waited.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4); }

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

template <int WF, int XF, int OUT, bool GELU, int OFMT>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  constexpr int kLayout = OUT == kOutMx ? kLayoutMx : kLayoutContig;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * kTileM, n0 = tn * kTileN;
  const int nk = (g.K + kTileStageK - 1) / kTileStageK;
  const int gx0 = m0 / kTileGroupRows, gw0 = n0 / kTileGroupRows;

  // ---- DMA sources.  Each wave copies 6 KB of each operand's 24 KB stage run
  // (1 KB per instruction, 16 bytes per lane) and 256 bytes of each 1 KB scale
  // run (4 bytes per lane).  Groups past the operand's last one (ragged tiles)
  // re-read its last group; those rows are never stored.
  uint32_t xo[kCodeCopiesPerWave], wo[kCodeCopiesPerWave];
#pragma unroll
  for (int i = 0; i < kCodeCopiesPerWave; ++i) {
    const int off = (wave * kCodeCopiesPerWave + i) * 1024 + lane * 16;
    const int grp = off / kChunkCodes, within = off - grp * kChunkCodes;
    xo[i] = (uint32_t)min(gx0 + grp, g.gx - 1) * kChunkCodes + within;
    wo[i] = (uint32_t)min(gw0 + grp, g.gw - 1) * kChunkCodes + within;
  }
  uint32_t xso, wso;
  {
    const int off = wave * 256 + lane * 4;
    const int grp = off / kChunkScales, within = off - grp * kChunkScales;
    xso = (uint32_t)min(gx0 + grp, g.gx - 1) * kChunkScales + within;
    wso = (uint32_t)min(gw0 + grp, g.gw - 1) * kChunkScales + within;
  }
  const int64_t x_stage = (int64_t)g.gx * kChunkCodes, w_stage = (int64_t)g.gw * kChunkCodes;
  const int64_t xs_stage = (int64_t)g.gx * kChunkScales, ws_stage = (int64_t)g.gw * kChunkScales;

  // copy number idx (0..13) of this wave's share of stage ks into ring slot `slot`
  auto issue_one = [&](int idx, int ks, int slot) {
    uint8_t* base = lds + slot * kSlotBytes;
    if (idx < kCodeCopiesPerWave) {
      __builtin_amdgcn_global_load_lds(g.x_codes + ks * x_stage + xo[idx],
                                       (lds_void_t*)(base + kOffX + (wave * kCodeCopiesPerWave + idx) * 1024), 16, 0,
                                       0);
    } else if (idx < 2 * kCodeCopiesPerWave) {
      const int i = idx - kCodeCopiesPerWave;
      __builtin_amdgcn_global_load_lds(g.w_codes + ks * w_stage + wo[i],
                                       (lds_void_t*)(base + kOffW + (wave * kCodeCopiesPerWave + i) * 1024), 16, 0, 0);
    } else if (idx == 2 * kCodeCopiesPerWave) {
      __builtin_amdgcn_global_load_lds(g.x_scales + ks * xs_stage + xso, (lds_void_t*)(base + kOffXs + wave * 256), 4,
                                       0, 0);
    } else {
      __builtin_amdgcn_global_load_lds(g.w_scales + ks * ws_stage + wso, (lds_void_t*)(base + kOffWs + wave * 256), 4,
                                       0, 0);
    }
  };
  auto issue = [&](int ks, int slot) {
#pragma unroll
    for (int i = 0; i < kCopiesPerStage; ++i) issue_one(i, ks, slot);
  };

  // ---- per-lane LDS read offsets for the MFMA operands
  const int wn = wave & 1, wm = wave >> 1;
  const int h = lane >> 5, j = lane & 31;
  const int wrow = feature_of_row<kLayout>(j);
  int w_off[4], x_off[4], ws_off[4], xs_off[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    w_off[f] = kOffW + (wn * 4 + f) * kChunkCodes + 3 * h * 512 + wrow * 16;
    x_off[f] = kOffX + (wm * 4 + f) * kChunkCodes + 3 * h * 512 + j * 16;
    ws_off[f] = kOffWs + (wn * 4 + f) * kChunkScales + wrow * 4 + 2 * h;
    xs_off[f] = kOffXs + (wm * 4 + f) * kChunkScales + j * 4 + 2 * h;
  }

  v16f acc[4][4];
#pragma unroll
  for (int fn = 0; fn < 4; ++fn)
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fn][fm][r] = 0.0f;

  // pieces 3h, 3h+1, 3h+2 of a row (48 bytes) -> the 6-dword operands of sub-steps 0 and 1
  auto read_operands = [](const uint8_t* p, v8i& s0, v8i& s1) {
    const u32x4 d0 = *reinterpret_cast<const u32x4*>(p);
    const u32x4 d1 = *reinterpret_cast<const u32x4*>(p + 512);
    const u32x4 d2 = *reinterpret_cast<const u32x4*>(p + 1024);
    s0 = v8i{(int)d0[0], (int)d0[1], (int)d0[2], (int)d0[3], (int)d1[0], (int)d1[1], 0, 0};
    s1 = v8i{(int)d1[2], (int)d1[3], (int)d2[0], (int)d2[1], (int)d2[2], (int)d2[3], 0, 0};
  };

  // One stage: read this lane's operands, then 32 MFMAs.  With COPY, the 14
  // copies of a later stage are interleaved one after every second MFMA: the
  // vector-memory address path then works beside the matrix cores instead of
  // holding up the first MFMAs of the stage behind a burst of copies.
  auto compute = [&](auto copy_tag, int slot, int ks2, int slot2) {
    constexpr bool COPY = decltype(copy_tag)::value;
    const uint8_t* st = lds + slot * kSlotBytes;
    v8i wa0, wa1, wb0, wb1, wc0, wc1, wd0, wd1;
    v8i xa0, xa1, xb0, xb1, xc0, xc1, xd0, xd1;
    read_operands(st + w_off[0], wa0, wa1);
    read_operands(st + x_off[0], xa0, xa1);
    read_operands(st + w_off[1], wb0, wb1);
    read_operands(st + x_off[1], xb0, xb1);
    read_operands(st + w_off[2], wc0, wc1);
    read_operands(st + x_off[2], xc0, xc1);
    read_operands(st + w_off[3], wd0, wd1);
    read_operands(st + x_off[3], xd0, xd1);
    const int ws0 = *reinterpret_cast<const uint16_t*>(st + ws_off[0]);
    const int ws1 = *reinterpret_cast<const uint16_t*>(st + ws_off[1]);
    const int ws2 = *reinterpret_cast<const uint16_t*>(st + ws_off[2]);
    const int ws3 = *reinterpret_cast<const uint16_t*>(st + ws_off[3]);
    const int xs0 = *reinterpret_cast<const uint16_t*>(st + xs_off[0]);
    const int xs1 = *reinterpret_cast<const uint16_t*>(st + xs_off[1]);
    const int xs2 = *reinterpret_cast<const uint16_t*>(st + xs_off[2]);
    const int xs3 = *reinterpret_cast<const uint16_t*>(st + xs_off[3]);
#define MXG_MFMA(FN, FM, W, X, WS, XS, S) \
  acc[FN][FM] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(W, X, acc[FN][FM], WF, XF, S, WS, S, XS)
#define MXG_COPY(I) \
  if constexpr (COPY && (I) < kCopiesPerStage) issue_one(I, ks2, slot2)
#define MXG_ROW(FN, W, WS, S, I0)                                                   \
  MXG_MFMA(FN, 0, W, xa##S, WS, xs0, S);                                           \
  MXG_MFMA(FN, 1, W, xb##S, WS, xs1, S);                                           \
  MXG_COPY(I0);                                                                    \
  MXG_MFMA(FN, 2, W, xc##S, WS, xs2, S);                                           \
  MXG_MFMA(FN, 3, W, xd##S, WS, xs3, S);                                           \
  MXG_COPY(I0 + 1)
    MXG_ROW(0, wa0, ws0, 0, 0);
    MXG_ROW(1, wb0, ws1, 0, 2);
    MXG_ROW(2, wc0, ws2, 0, 4);
    MXG_ROW(3, wd0, ws3, 0, 6);
    MXG_ROW(0, wa1, ws0, 1, 8);
    MXG_ROW(1, wb1, ws1, 1, 10);
    MXG_ROW(2, wc1, ws2, 1, 12);
    MXG_ROW(3, wd1, ws3, 1, 14);
#undef MXG_ROW
#undef MXG_COPY
#undef MXG_MFMA
    if constexpr (COPY) {
      // all LDS reads first, then {2 MFMA, 1 copy} x 14, then the last 4 MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 32, 0);
#pragma unroll
      for (int i = 0; i < kCopiesPerStage; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 32 - 2 * kCopiesPerStage, 0);
    }
  };
  using with_copies = std::integral_constant<bool, true>;
  using no_copies = std::integral_constant<bool, false>;

  // ---- main loop over the ring.  At the top of step ks the copies of stages
  // ks and ks+1 are in flight; waiting until at most one stage's copies are
  // outstanding (they complete in order) means stage ks has landed, and the
  // barrier makes every wave's part of it visible and retires the reads of the
  // slot that stage ks+2 is about to overwrite.  The last two steps are peeled
  // so the steady-state body is one basic block.
  if (nk > 0) issue(0, 0);
  if (nk > 1) issue(1, 1);
  int ks = 0, slot = 0;
  for (; ks + 2 < nk; ++ks) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kCopiesPerStage));
    __builtin_amdgcn_s_barrier();
    compute(with_copies{}, slot, ks + 2, slot == 0 ? 2 : slot - 1);
    __builtin_amdgcn_sched_barrier(0);
    slot = slot == 2 ? 0 : slot + 1;
  }
  if (ks + 1 < nk) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kCopiesPerStage));
    __builtin_amdgcn_s_barrier();
    compute(no_copies{}, slot, 0, 0);
    slot = slot == 2 ? 0 : slot + 1;
    ++ks;
  }
  if (ks < nk) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    compute(no_copies{}, slot, 0, 0);
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
        const int nb = (nw0 + fn * 32) / 32;  // 32-feature block of this fragment
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
        uint32_t sbyte = sc.byte;
        if (sc.nonfinite) q = v6u{0, 0, 0, 0, 0, 0};
        const int gm = (mw0 + fm * 32) / kTileGroupRows;
        const int stage = nb >> 2, qb = nb & 3;
        if (gm < g.gx && stage < (g.N + kTileStageK - 1) / kTileStageK) {
          if (m >= g.M || nb >= g.N / 32) {  // layout padding
            q = v6u{0, 0, 0, 0, 0, 0};
            sbyte = 127u;
          }
          uint8_t* chunk = static_cast<uint8_t*>(g.out) + ((int64_t)stage * g.gx + gm) * kChunkCodes;
          const int o = 24 * qb + 12 * h;  // this lane's 12 bytes of the row's 96-byte slice
#pragma unroll
          for (int d = 0; d < 3; ++d) {
            const int od4 = o + 4 * d;
            *reinterpret_cast<uint32_t*>(chunk + (od4 >> 4) * 512 + j * 16 + (od4 & 15)) = q[d];
          }
          if (h == 0)
            g.out_scales[((int64_t)stage * g.gx + gm) * kChunkScales + j * 4 + qb] = (uint8_t)sbyte;
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
              for (int q4 = 0; q4 < 4; ++q4)
                o[q4] = u32x4{__float_as_uint(v[4 * q4]), __float_as_uint(v[4 * q4 + 1]),
                              __float_as_uint(v[4 * q4 + 2]), __float_as_uint(v[4 * q4 + 3])};
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
hipError_t launch_variant(const GemmArgs& a, int epilogue, int out_kind, int out_fmt, hipStream_t stream) {
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
  } else if (out_fmt == kFmtE2M3) {
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
  return hipGetLastError();
}

}  // namespace

// One translation unit per (weight, activation) format pair, so the variants
// build in parallel.
template <int WF, int XF>
hipError_t launch_gemm_formats(const GemmArgs& a, int epilogue, int out_kind, int out_fmt, hipStream_t stream) {
  return launch_variant<WF, XF>(a, epilogue, out_kind, out_fmt, stream);
}

}  // namespace mxg
