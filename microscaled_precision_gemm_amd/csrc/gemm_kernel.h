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
//    a ring of 3 slots.  The waits on those copies are explicit (s_waitcnt
//    vmcnt) and the barrier is a bare s_barrier, so a stage only waits for its
//    own data.
//  * Inside a stage, lane half h of sub-step s handles K-block 2h + s (the K
//    order inside one accumulation is free as long as both operands agree).
//    The layout's planes make each sub-step operand one 16-byte and one
//    8-byte LDS read into adjacent registers, conflict-free (the 32 lanes of a
//    half read 512 or 256 consecutive bytes), with one 16-bit scale pair per
//    fragment; op_sel = s picks the byte.
//  * Operand registers are double buffered per half stage: the MFMAs of one
//    sub-step run while the operands of the next are read from LDS, and the
//    copies of stage ks+3 are interleaved one per MFMA into the slot stage ks
//    came from, so the LDS, the address path and the matrix cores overlap.
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

// Tile order.  With xcd_remap, workgroup b (dispatched round-robin to XCD
// b % 8) takes position b / 8 of a contiguous range per XCD, so the tiles one
// XCD has in flight are neighbours; positions then walk a grouped order,
// group_m m-tiles wide, so that those neighbours share A and W stages in the
// XCD's L2.
__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int group_m, int xcd_remap, int& tm,
                                            int& tn) {
  const int total = tiles_m * tiles_n;
  int s = b;
  if (xcd_remap && total >= 64) {
    const int xcd = b & 7, idx = b >> 3;
    const int per = total >> 3, rem = total & 7;
    s = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  }
  const int group = s / (group_m * tiles_n);
  const int first_m = group * group_m;
  const int gsize = min(tiles_m - first_m, group_m);
  const int in = s - group * group_m * tiles_n;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

// Eight v_permlane32_swap_b32: after it, a[i] holds a[i] of lanes 0..31 in
// lanes 0..31 and b[i] of lanes 0..31 in lanes 32..63, b[i] holds a[i] of lanes
// 32..63 in lanes 0..31 and b[i] of lanes 32..63 in lanes 32..63.  On gfx950 a
// swap issued right after a VALU write of one of its operands reads stale
// lanes, and the compiler does not put wait states in between, so the swaps
// are written out with s_nop 4 ahead of them (the same wait is not needed
// before a VALU reads their results).
__device__ __forceinline__ void swap_halves8(uint32_t (&a)[8], uint32_t (&b)[8]) {
  asm volatile(
      "s_nop 4\n\t"
      "v_permlane32_swap_b32 %0, %8\n\t"
      "v_permlane32_swap_b32 %1, %9\n\t"
      "v_permlane32_swap_b32 %2, %10\n\t"
      "v_permlane32_swap_b32 %3, %11\n\t"
      "v_permlane32_swap_b32 %4, %12\n\t"
      "v_permlane32_swap_b32 %5, %13\n\t"
      "v_permlane32_swap_b32 %6, %14\n\t"
      "v_permlane32_swap_b32 %7, %15"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7]),
        "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5]), "+v"(b[6]), "+v"(b[7]));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &a, 2);
  __builtin_memcpy(&ub, &b, 2);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

template <int WF, int XF, int OUT, int EPI, int OFMT>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  constexpr int kLayout = OUT == kOutMx ? kLayoutMx : kLayoutContig;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, g.group_m, g.xcd_remap, tm, tn);
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

  // ---- per-lane LDS bases in ring slot 0; fragment f (32 rows) adds
  // f * kChunkCodes.  Half h of a chunk holds this lane's blocks 2h (sub-step
  // 0: plane A + plane L) and 2h+1 (sub-step 1: plane H + plane B).
  const int wn = wave & 1, wm = wave >> 1;
  const int h = lane >> 5, j = lane & 31;
  const int wrow = feature_of_row<kLayout>(j);
  const int w16 = kOffW + wn * 4 * kChunkCodes + h * kHalfBytes + wrow * 16;
  const int x16 = kOffX + wm * 4 * kChunkCodes + h * kHalfBytes + j * 16;
  const int w8 = kOffW + wn * 4 * kChunkCodes + h * kHalfBytes + wrow * 8;
  const int x8 = kOffX + wm * 4 * kChunkCodes + h * kHalfBytes + j * 8;
  const int wsc = kOffWs + wn * 4 * kChunkScales + wrow * 4 + 2 * h;
  const int xsc = kOffXs + wm * 4 * kChunkScales + j * 4 + 2 * h;

  v16f acc[4][4];
#pragma unroll
  for (int fn = 0; fn < 4; ++fn)
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fn][fm][r] = 0.0f;

  // One sub-step operand is a 16-byte and an 8-byte LDS read landing in
  // adjacent registers (the MFMA reads 6 of the 8).  The 8-byte reads are
  // volatile so they are not fused into one 16-byte read whose halves would
  // belong to different operands (that costs register moves).
  typedef const volatile __attribute__((address_space(3))) u32x2 lds_u32x2_t;
  auto rd16 = [&](int off) { return *reinterpret_cast<const u32x4*>(lds + off); };
  auto rd8 = [&](int off) { return (u32x2)(*(lds_u32x2_t*)(lds + off)); };
  auto op0 = [&](int b16, int b8) {
    const u32x4 a = rd16(b16 + kPlaneA);
    const u32x2 c = rd8(b8 + kPlaneL);
    return v8i{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], 0, 0};
  };
  auto op1 = [&](int b16, int b8) {
    const u32x2 c = rd8(b8 + kPlaneH);
    const u32x4 a = rd16(b16 + kPlaneB);
    return v8i{(int)c[0], (int)c[1], (int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0};
  };
  struct Half {  // one sub-step's operands: 4 weight and 4 activation fragments
    v8i w0, w1, w2, w3, x0, x1, x2, x3;
  };
  struct Scales {  // scale byte pairs (blocks 2h, 2h+1) of the 8 fragments
    int w0, w1, w2, w3, x0, x1, x2, x3;
  };
  auto read_half = [&](int sl, auto sub_tag) {
    constexpr int SUB = decltype(sub_tag)::value;
    const int so = sl * kSlotBytes;
    auto op = [&](int b16, int b8, int f) {
      return SUB == 0 ? op0(so + b16 + f * kChunkCodes, so + b8 + f * kChunkCodes)
                      : op1(so + b16 + f * kChunkCodes, so + b8 + f * kChunkCodes);
    };
    Half r;
    r.w0 = op(w16, w8, 0);
    r.x0 = op(x16, x8, 0);
    r.w1 = op(w16, w8, 1);
    r.x1 = op(x16, x8, 1);
    r.w2 = op(w16, w8, 2);
    r.x2 = op(x16, x8, 2);
    r.w3 = op(w16, w8, 3);
    r.x3 = op(x16, x8, 3);
    return r;
  };
  auto scale_at = [&](int so, int base, int f) {
    return (int)*reinterpret_cast<const uint16_t*>(lds + so + base + f * kChunkScales);
  };
  auto read_scales = [&](int sl) {
    const int so = sl * kSlotBytes;
    Scales c;
    c.w0 = scale_at(so, wsc, 0);
    c.w1 = scale_at(so, wsc, 1);
    c.w2 = scale_at(so, wsc, 2);
    c.w3 = scale_at(so, wsc, 3);
    c.x0 = scale_at(so, xsc, 0);
    c.x1 = scale_at(so, xsc, 1);
    c.x2 = scale_at(so, xsc, 2);
    c.x3 = scale_at(so, xsc, 3);
    return c;
  };
#define MXG_MFMA(FN, FM, S) \
  acc[FN][FM] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(r.w##FN, r.x##FM, acc[FN][FM], WF, XF, S, c.w##FN, S, c.x##FM)
  // the 16 MFMAs of one sub-step
  auto mfmas = [&](const Half& r, const Scales& c, auto sub_tag) {
    constexpr int S = decltype(sub_tag)::value;
    MXG_MFMA(0, 0, S); MXG_MFMA(0, 1, S); MXG_MFMA(0, 2, S); MXG_MFMA(0, 3, S);
    MXG_MFMA(1, 0, S); MXG_MFMA(1, 1, S); MXG_MFMA(1, 2, S); MXG_MFMA(1, 3, S);
    MXG_MFMA(2, 0, S); MXG_MFMA(2, 1, S); MXG_MFMA(2, 2, S); MXG_MFMA(2, 3, S);
    MXG_MFMA(3, 0, S); MXG_MFMA(3, 1, S); MXG_MFMA(3, 2, S); MXG_MFMA(3, 3, S);
  };
  // The steady-state phases, written in issue order (the LDS reads and the
  // copies into LDS keep their program order).  Each stage's 14 copies are
  // split: copies 0..6 of stage ks+3 go out in phase 1 of stage ks (into the
  // slot stage ks has just been read from), copies 7..13 in phase 0 of stage
  // ks+1, so the vector-memory path sees 7 copies per 16 MFMAs throughout.
  // Phase 1: sub-step 1 MFMAs, reads of the next stage's sub-step 0 operands
  // and scales, first half of stage ks2's copies into slot slot2.
  auto phase1 = [&](const Half& r, const Scales& c, int ks2, int slot2, int nsl, Half& nr, Scales& ns) {
    const int so = nsl * kSlotBytes;
#define MXG_RD(DST, B16, B8, F) nr.DST = op0(so + B16 + (F) * kChunkCodes, so + B8 + (F) * kChunkCodes)
    MXG_MFMA(0, 0, 1); MXG_RD(w0, w16, w8, 0); issue_one(0, ks2, slot2);
    MXG_MFMA(0, 1, 1); MXG_RD(x0, x16, x8, 0);
    MXG_MFMA(0, 2, 1); MXG_RD(w1, w16, w8, 1); issue_one(1, ks2, slot2);
    MXG_MFMA(0, 3, 1); MXG_RD(x1, x16, x8, 1);
    MXG_MFMA(1, 0, 1); MXG_RD(w2, w16, w8, 2); issue_one(2, ks2, slot2);
    MXG_MFMA(1, 1, 1); MXG_RD(x2, x16, x8, 2);
    MXG_MFMA(1, 2, 1); MXG_RD(w3, w16, w8, 3); issue_one(3, ks2, slot2);
    MXG_MFMA(1, 3, 1); MXG_RD(x3, x16, x8, 3);
    MXG_MFMA(2, 0, 1); ns.w0 = scale_at(so, wsc, 0); ns.w1 = scale_at(so, wsc, 1); issue_one(4, ks2, slot2);
    MXG_MFMA(2, 1, 1); ns.w2 = scale_at(so, wsc, 2); ns.w3 = scale_at(so, wsc, 3);
    MXG_MFMA(2, 2, 1); ns.x0 = scale_at(so, xsc, 0); ns.x1 = scale_at(so, xsc, 1); issue_one(5, ks2, slot2);
    MXG_MFMA(2, 3, 1); ns.x2 = scale_at(so, xsc, 2); ns.x3 = scale_at(so, xsc, 3);
    MXG_MFMA(3, 0, 1); issue_one(6, ks2, slot2);
    MXG_MFMA(3, 1, 1);
    MXG_MFMA(3, 2, 1);
    MXG_MFMA(3, 3, 1);
    // pin that order for the scheduler
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
#undef MXG_RD
  };
  // phase 0 with the second half (copies 7..13) of stage ks2 interleaved
  auto phase0 = [&](const Half& r, const Scales& c, int sl, Half& nr, int ks2, int slot2) {
    const int so = sl * kSlotBytes;
#define MXG_RD1(DST, B16, B8, F) nr.DST = op1(so + B16 + (F) * kChunkCodes, so + B8 + (F) * kChunkCodes)
    MXG_MFMA(0, 0, 0); MXG_RD1(w0, w16, w8, 0);
    MXG_MFMA(0, 1, 0); MXG_RD1(x0, x16, x8, 0); issue_one(7, ks2, slot2);
    MXG_MFMA(0, 2, 0); MXG_RD1(w1, w16, w8, 1);
    MXG_MFMA(0, 3, 0); MXG_RD1(x1, x16, x8, 1); issue_one(8, ks2, slot2);
    MXG_MFMA(1, 0, 0); MXG_RD1(w2, w16, w8, 2);
    MXG_MFMA(1, 1, 0); MXG_RD1(x2, x16, x8, 2); issue_one(9, ks2, slot2);
    MXG_MFMA(1, 2, 0); MXG_RD1(w3, w16, w8, 3);
    MXG_MFMA(1, 3, 0); MXG_RD1(x3, x16, x8, 3); issue_one(10, ks2, slot2);
    MXG_MFMA(2, 0, 0);
    MXG_MFMA(2, 1, 0); issue_one(11, ks2, slot2);
    MXG_MFMA(2, 2, 0);
    MXG_MFMA(2, 3, 0); issue_one(12, ks2, slot2);
    MXG_MFMA(3, 0, 0);
    MXG_MFMA(3, 1, 0); issue_one(13, ks2, slot2);
    MXG_MFMA(3, 2, 0);
    MXG_MFMA(3, 3, 0);
#undef MXG_RD1
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };
#undef MXG_MFMA
  static_assert(kCopiesPerStage == 14, "the phases interleave 7 + 7 copies");
  auto next_slot = [](int sl) { return sl == 2 ? 0 : sl + 1; };
  using sub0 = std::integral_constant<int, 0>;
  using sub1 = std::integral_constant<int, 1>;

  // ---- main loop over the 3-slot ring, with the operand registers double
  // buffered at half-stage granularity.  At the top of stage ks the lane holds
  // stage ks's sub-step 0 operands (ra) and scales (sc); all copies of stage
  // ks+1 and the first half of stage ks+2's are in flight.  Phase 0: sub-step
  // 0 MFMAs while reading stage ks's sub-step 1 operands (rb) and issuing the
  // second half of stage ks+2's copies.  Then wait until at most one stage's
  // copies are outstanding (they complete in order: stage ks+1 has landed),
  // and barrier: every wave's part of stage ks+1 is visible and every wave is
  // done reading slot ks.  Phase 1: sub-step 1 MFMAs while reading stage
  // ks+1's sub-step 0 operands and scales and issuing the first half of stage
  // ks+3's copies into slot ks.
  auto issue_half = [&](int ks2, int sl2, int first) {
#pragma unroll
    for (int i = 0; i < 7; ++i) issue_one(first + i, ks2, sl2);
  };
  if (nk > 0) issue(0, 0);
  if (nk > 1) issue(1, 1);
  if (nk > 2) issue_half(2, 2, 0);
  if (nk > 2)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kCopiesPerStage + 7));
  else if (nk > 1)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kCopiesPerStage));
  else
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __builtin_amdgcn_s_barrier();
  Half ra = read_half(0, sub0{});
  Scales sc = read_scales(0);
  int ks = 0, slot = 0;
  for (; ks + 3 < nk; ++ks) {
    const int nsl = next_slot(slot);
    Half rb;
    phase0(ra, sc, slot, rb, ks + 2, next_slot(nsl));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kCopiesPerStage));
    __builtin_amdgcn_s_barrier();
    Scales sn;
    phase1(rb, sc, ks + 3, slot, nsl, ra, sn);
    __builtin_amdgcn_sched_barrier(0);
    sc = sn;
    slot = nsl;
  }
  for (; ks < nk; ++ks) {
    const int nsl = next_slot(slot);
    if (ks + 2 < nk) issue_half(ks + 2, next_slot(nsl), 7);
    const Half rb = read_half(slot, sub1{});
    mfmas(ra, sc, sub0{});
    Scales sn = sc;
    if (ks + 1 < nk) {
      if (ks + 2 < nk)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kCopiesPerStage));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
      __builtin_amdgcn_s_barrier();
      ra = read_half(nsl, sub0{});
      sn = read_scales(nsl);
    }
    mfmas(rb, sc, sub1{});
    sc = sn;
    slot = nsl;
  }

  // ---- epilogue
  const int mw0 = m0 + wm * 128, nw0 = n0 + wn * 128;
  // SwiGLU: this wave's 128 stacked rows are the gate rows (fragments 0, 1)
  // and the up rows (fragments 2, 3) of output features nw0/2 .. nw0/2 + 63.
  constexpr bool kSwiglu = EPI == kEpiSwiglu;
  const int n_out = kSwiglu ? g.N / 2 : g.N;
  auto act = [&](float x) { return EPI == kEpiGeluTanh ? gelu_tanh_f32(x) : x; };
  if constexpr (OUT == kOutMx) {
    // MX output along N.  A pair of fragment values (va, vb) holds two
    // consecutive 32-feature blocks of one 128-feature output stage; each
    // lane has 16 features of each, and one permlane32 swap per register
    // gathers the first block in lanes 0..31 and the second in lanes 32..63,
    // so every lane owns one whole block of token j: its amax is lane-local,
    // one 32-value conversion covers it, and its 24 code bytes are one
    // 16-byte and one 8-byte run of the tiled layout.
    const int n_stages = (n_out + kTileStageK - 1) / kTileStageK;
    auto emit_pair = [&](const v16f& va, const v16f& vb, int m, int gm, int stage, int pr) {
      // lo: features 0..15 of this lane's block (even ones in 0..7, odd in
      // 8..15), hi: features 16..31 in the same order
      v16f lo, hi;
#pragma unroll
      for (int half8 = 0; half8 < 2; ++half8) {
        uint32_t x[8], y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          x[i] = __float_as_uint(va[8 * half8 + i]);
          y[i] = __float_as_uint(vb[8 * half8 + i]);
        }
        swap_halves8(x, y);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          lo[8 * half8 + i] = __uint_as_float(x[i]);
          hi[8 * half8 + i] = __uint_as_float(y[i]);
        }
      }
      uint32_t amax = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t x = __float_as_uint(lo[r]) & 0x7fffffffu, y = __float_as_uint(hi[r]) & 0x7fffffffu;
        const uint32_t xy = x > y ? x : y;
        amax = xy > amax ? xy : amax;
      }
      const BlockScale sc = scale_from_f32_bits<OFMT>(amax);
      v16f ev, od;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ev[i] = lo[i];
        ev[8 + i] = hi[i];
        od[i] = lo[8 + i];
        od[8 + i] = hi[8 + i];
      }
      v6u q = cvt_f32x2x16<OFMT>(ev, od, sc.scale);
      uint32_t sbyte = sc.byte;
      if (sc.nonfinite) q = v6u{0, 0, 0, 0, 0, 0};
      const int qb = 2 * pr + h;  // this lane's block within the stage
      const int nb = stage * 4 + qb;
      if (gm < g.gx && stage < n_stages) {
        if (m >= g.M || nb >= n_out / 32) {  // layout padding
          q = v6u{0, 0, 0, 0, 0, 0};
          sbyte = 127u;
        }
        // even block: plane A (bytes 0..15) + plane L (16..23);
        // odd block: plane H (bytes 0..7) + plane B (8..23)
        uint8_t* half = static_cast<uint8_t*>(g.out) + ((int64_t)stage * g.gx + gm) * kChunkCodes + pr * kHalfBytes;
        const u32x4 d16 = h == 0 ? u32x4{q[0], q[1], q[2], q[3]} : u32x4{q[2], q[3], q[4], q[5]};
        const u32x2 d8 = h == 0 ? u32x2{q[4], q[5]} : u32x2{q[0], q[1]};
        *reinterpret_cast<u32x4*>(half + (h == 0 ? kPlaneA : kPlaneB) + j * 16) = d16;
        *reinterpret_cast<u32x2*>(half + (h == 0 ? kPlaneL : kPlaneH) + j * 8) = d8;
        g.out_scales[((int64_t)stage * g.gx + gm) * kChunkScales + j * 4 + qb] = (uint8_t)sbyte;
      }
    };
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
      const int m = mw0 + fm * 32 + j;
      const int gm = (mw0 + fm * 32) / kTileGroupRows;
      if constexpr (kSwiglu) {
        // output features nw0/2 .. +63: blocks 2p, 2p+1 of stage nw0/256, p = (nw0/128) % 2
        v16f va, vb;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          va[r] = silu_f32(acc[0][fm][r]) * acc[2][fm][r];
          vb[r] = silu_f32(acc[1][fm][r]) * acc[3][fm][r];
        }
        emit_pair(va, vb, m, gm, nw0 / (2 * kTileStageK), (nw0 / kTileStageK) & 1);
      } else {
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          v16f va = acc[2 * pr][fm], vb = acc[2 * pr + 1][fm];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            va[r] = act(va[r]);
            vb[r] = act(vb[r]);
          }
          emit_pair(va, vb, m, gm, nw0 / kTileStageK, pr);
        }
      }
    }
    return;
  }
  constexpr int kOutFrags = kSwiglu ? 2 : 4;
#pragma unroll
  for (int fn = 0; fn < kOutFrags; ++fn) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
      const int m = mw0 + fm * 32 + j;
      v16f v;
      if constexpr (kSwiglu) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = silu_f32(acc[fn][fm][r]) * acc[fn + 2][fm][r];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = act(acc[fn][fm][r]);
      }
      {
        const int n = (kSwiglu ? nw0 / 2 : nw0) + fn * 32 + 16 * h;
        if (m < g.M) {
          if constexpr (OUT == kOutBf16) {
            uint16_t* out = static_cast<uint16_t*>(g.out) + (int64_t)m * g.ldo;
            if (g.vec_store && n + 16 <= n_out) {
              u32x4* o = reinterpret_cast<u32x4*>(out + n);
              o[0] = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                           pack_bf16x2(v[6], v[7])};
              o[1] = u32x4{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
                           pack_bf16x2(v[14], v[15])};
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (n + r < n_out) {
                  const __bf16 b = (__bf16)v[r];
                  __builtin_memcpy(out + n + r, &b, 2);
                }
            }
          } else {
            float* out = static_cast<float*>(g.out) + (int64_t)m * g.ldo;
            if (g.vec_store && n + 16 <= n_out) {
              u32x4* o = reinterpret_cast<u32x4*>(out + n);
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4)
                o[q4] = u32x4{__float_as_uint(v[4 * q4]), __float_as_uint(v[4 * q4 + 1]),
                              __float_as_uint(v[4 * q4 + 2]), __float_as_uint(v[4 * q4 + 3])};
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (n + r < n_out) out[n + r] = v[r];
            }
          }
        }
      }
    }
  }
}

template <int WF, int XF, int EPI>
void launch_epi(const GemmArgs& a, int out_kind, int out_fmt, dim3 grid, dim3 block, hipStream_t stream) {
  if (out_kind == kOutF32)
    hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutF32, EPI, kFmtE2M3>), grid, block, 0, stream, a);
  else if (out_kind == kOutBf16)
    hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutBf16, EPI, kFmtE2M3>), grid, block, 0, stream, a);
  else if (out_fmt == kFmtE2M3)
    hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutMx, EPI, kFmtE2M3>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutMx, EPI, kFmtE3M2>), grid, block, 0, stream, a);
}

template <int WF, int XF>
hipError_t launch_variant(const GemmArgs& a, int epilogue, int out_kind, int out_fmt, hipStream_t stream) {
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(kThreads);
  if (epilogue == kEpiGeluTanh)
    launch_epi<WF, XF, kEpiGeluTanh>(a, out_kind, out_fmt, grid, block, stream);
  else if (epilogue == kEpiSwiglu)
    launch_epi<WF, XF, kEpiSwiglu>(a, out_kind, out_fmt, grid, block, stream);
  else
    launch_epi<WF, XF, kEpiNone>(a, out_kind, out_fmt, grid, block, stream);
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
