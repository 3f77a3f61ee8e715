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
//    FP6 codes in 6 VGPRs and one E8M0 byte picked by op_sel); the launch
//    configuration can instead pick 256 x 128 tiles (two workgroups per CU)
//    or 8 waves of 128 x 64 per 256 x 256 tile (see Ring).  The same
//    kernel takes the instruction's other operand formats (FP4 E2M1 in 4
//    VGPRs, FP8 E4M3 / E5M2 in 8), the layout's chunk size and the ring depth
//    following the element width.
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

constexpr int kGroupsPerTile = kTileM / kTileGroupRows;            // 8 activation groups per tile
constexpr int kStageScales = kGroupsPerTile * kChunkScales;         // 1 KB of activation scales
static_assert(kStageScales == 4 * 64 * 4, "one 4-byte copy per lane per wave covers a stage's scales");

// LDS ring and copy schedule for weight format WF and activation format XF.
// A slot holds one stage of both operands (256 rows x 128 K each, 4 KB per
// element bit) and their scales; three slots when they fit in the 160 KB of
// LDS, else two.  Each wave copies 1 KB per instruction (16 bytes per lane);
// with 4 waves and 256 weight rows that is bits(XF) activation copies,
// bits(WF) weight copies and one scale copy per operand per stage.  With three slots, stage ks+3's copies go out half in
// phase 1 of stage ks and half in phase 0 of stage ks+1; with two, stage
// ks+2's copies all go out in phase 1 of stage ks (the slot it refills is
// free from the middle of stage ks on, and the copies have a whole stage of
// matrix work to land).
//
// TN is the tile's width in weight rows (output features, or for SwiGLU
// stacked gate/up rows): 256 (4 waves of 128 x 128, 256 accumulator
// registers each, one workgroup per CU) or 128 (4 waves of 128 x 64, 128
// accumulators, and a two-slot ring of 37.5 KB slots, so that two workgroups
// share a CU and one's waits, prologue and epilogue overlap the other's
// matrix work).  WV is the number of waves: 4 (2 x 2 waves over
// the tile) or, for TN = 256, 8 (2 x 4 waves of 128 x 64, two waves per
// SIMD sharing the three-slot ring; each wave issues half the copies, and
// its one scale copy is the activations' (waves 0-3) or the weights'
// (waves 4-7) 256-byte quarter).
template <int WF, int XF, int TN = 256, int WV = 4>
struct Ring {
  static constexpr int kWaves = WV, kThreads = 64 * WV;
  static constexpr int kWN = WV / 2;                                  // waves along N (2 along M)
  static constexpr int kBW = fmt_bits(WF), kBX = fmt_bits(XF);
  static constexpr int kChunkW = chunk_codes(kBW), kChunkX = chunk_codes(kBX);
  static constexpr int kHalfW = half_codes(kBW), kHalfX = half_codes(kBX);
  static constexpr int kGroupsW = TN / kTileGroupRows;                // weight groups per tile
  static constexpr int kFW = TN / kWN / 32;                           // weight fragments per wave
  static constexpr int kMfmaPhase = 4 * kFW;                          // MFMAs per sub-step
  static constexpr int kStageW = kGroupsW * kChunkW, kStageX = kGroupsPerTile * kChunkX;
  static constexpr int kStageScalesW = kGroupsW * kChunkScales;
  static constexpr int kOffX = 0;
  static constexpr int kOffW = kStageX;
  static constexpr int kOffXs = kStageX + kStageW;
  static constexpr int kOffWs = kOffXs + kStageScales;
  static constexpr int kSlot = kStageX + kStageW + kStageScales + kStageScalesW;  // 51200 for 6-bit, TN 256
  static constexpr int kSlots = TN == 256 && 3 * kSlot <= 160 * 1024 ? 3 : 2;
  static constexpr int kLds = kSlots * kSlot;
  static constexpr int kCX = kStageX / 1024 / WV, kCW = kStageW / 1024 / WV;  // 1 KB code copies per wave
  static constexpr int kScaleCopies = WV == 8 ? 1 : 2;                      // 256-byte scale copies per wave
  static constexpr int kCopies = kCX + kCW + kScaleCopies;
  static constexpr int kFirst = kSlots == 3 ? (kCopies + 1) / 2 : kCopies;  // issued in phase 1
  static constexpr int kSecond = kCopies - kFirst;                           // issued in phase 0
  static_assert(kLds <= 160 * 1024, "gfx950 LDS is 160 KB per workgroup");
  static_assert(TN == 256 || 2 * kLds <= 160 * 1024, "two TN = 128 workgroups share a CU's LDS");
  static_assert(kStageScalesW == 1024 || kStageScalesW == 512, "weight scales: 4 (or 2 duplicated) waves x 256 B");
  static_assert(kCopies + kFirst <= 63, "vmcnt counts at most 63 outstanding copies");
  static_assert(WV == 4 || (WV == 8 && TN == 256), "eight waves tile 256 x 256 as 2 x 4 waves of 128 x 64");
  static_assert(kStageX % (1024 * WV) == 0 && kStageW % (1024 * WV) == 0, "every wave copies whole 1 KB runs");
};

// MFMA (0 .. m-1) of a phase of m MFMAs after which copy c of n goes out:
// every other MFMA when they fit (phase 1 from the first, phase 0 from the
// second), spread evenly otherwise.
constexpr int copy_slot(int c, int n, int phase, int m) {
  return 2 * n <= m ? 2 * c + (phase == 0 ? 1 : 0) : c * m / n;
}
constexpr int copies_after(int i, int n, int phase, int m) {
  int k = 0;
  for (int c = 0; c < n; ++c) k += copy_slot(c, n, phase, m) == i;
  return k;
}
constexpr int first_copy_after(int i, int n, int phase, int m) {
  for (int c = 0; c < n; ++c)
    if (copy_slot(c, n, phase, m) == i) return c;
  return n;
}
// Phase 1's scale-pair reads: nf fragment reads go first, one per MFMA; the
// ns scale reads follow, two (or more, if the MFMAs run out) per MFMA.
constexpr int scales_per_mfma(int nf, int ns, int m) {
  return (ns + (m - nf) - 1) / (m - nf) > 2 ? (ns + (m - nf) - 1) / (m - nf) : 2;
}
constexpr int scale_reads_after(int i, int nf, int ns, int m) {
  const int per = scales_per_mfma(nf, ns, m);
  const int first = (i - nf) * per;
  return i < nf || first >= ns ? 0 : (ns - first < per ? ns - first : per);
}

template <int... I>
struct Seq {};
template <int N, int... I>
struct MakeSeq : MakeSeq<N - 1, N - 1, I...> {};
template <int... I>
struct MakeSeq<0, I...> {
  using type = Seq<I...>;
};
template <class F, int... I>
__device__ __forceinline__ void static_for(F&& f, Seq<I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N>
using SeqN = typename MakeSeq<N>::type;

// global -> LDS copies of 16 bytes (codes) and 4 bytes (scales) per lane.
// Kept out of the kernel template: the host compilation cannot check the
// target builtin once its arguments depend on template parameters, and then
// drops the kernel's launch stub.
__device__ __forceinline__ void copy16_to_lds(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
}
__device__ __forceinline__ void copy4_to_lds(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 4, 0, 0);
}

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

template <int WF, int XF, int OUT, int EPI, int OFMT, int TN = 256, int WV = 4>
__global__ __launch_bounds__(64 * WV, TN == 256 ? 1 : 2) void gemm_kernel(const GemmArgs g) {
  using R = Ring<WF, XF, TN, WV>;
  constexpr bool kSwiglu = EPI == kEpiSwiglu;
  // SwiGLU where a wave holds two weight fragments (128-feature tiles with 4
  // waves, 256-feature tiles with 8): each run of 128 weight rows is 64 gate
  // rows and the 64 up rows of the same features, so the wave takes gate group
  // g and up group 2 + g of one run (run wn / 2, g = wn % 2) as its two
  // fragments, 32 output features, and each gate value's up value is in the
  // same lane.  With four fragments per wave (256-feature tiles, 4 waves) the
  // wave's 128 rows are one whole run.
  constexpr bool kSwPair = kSwiglu && R::kFW == 2;
  constexpr bool kSwNarrow = kSwiglu && TN == 128;
  __shared__ __attribute__((aligned(16))) uint8_t lds[R::kLds];
  constexpr int kLayout = OUT == kOutMx ? kLayoutMx : kLayoutContig;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, g.group_m, g.xcd_remap, tm, tn);
  const int m0 = tm * kTileM, n0 = tn * TN;
  const int nk = (g.K + kTileStageK - 1) / kTileStageK;
  const int gx0 = m0 / kTileGroupRows, gw0 = n0 / kTileGroupRows;

  // ---- DMA sources.  Each wave copies a quarter of each operand's stage run
  // (1 KB per instruction, 16 bytes per lane) and 256 bytes of each 1 KB
  // scale run (4 bytes per lane).  Groups past the operand's last one (ragged
  // tiles) re-read its last group; those rows are never stored.
  uint32_t xo[R::kCX], wo[R::kCW];
#pragma unroll
  for (int i = 0; i < R::kCX; ++i) {
    const int off = (wave * R::kCX + i) * 1024 + lane * 16;
    const int grp = off / R::kChunkX, within = off - grp * R::kChunkX;
    xo[i] = (uint32_t)min(gx0 + grp, g.gx - 1) * R::kChunkX + within;
  }
#pragma unroll
  for (int i = 0; i < R::kCW; ++i) {
    const int off = (wave * R::kCW + i) * 1024 + lane * 16;
    const int grp = off / R::kChunkW, within = off - grp * R::kChunkW;
    wo[i] = (uint32_t)min(gw0 + grp, g.gw - 1) * R::kChunkW + within;
  }
  // scale copies: quarter q (256 bytes) of the activations' and of the
  // weights' 1 KB scale run of a stage (4 waves: quarter `wave` of both; 8
  // waves: waves 0-3 the activations', waves 4-7 the weights')
  const int xq = WV == 8 ? (wave & 3) : wave;
  const int wq = WV == 8 ? (wave & 3) : wave;
  uint32_t xso, wso;
  {
    const int off = xq * 256 + lane * 4;
    const int grp = off / kChunkScales, within = off - grp * kChunkScales;
    xso = (uint32_t)min(gx0 + grp, g.gx - 1) * kChunkScales + within;
    // TN = 128: a 512-byte weight scale run; waves 2 and 3 copy the same bytes
    // as waves 0 and 1 (identical data), so every wave issues the same copies
    const int woff = (R::kStageScalesW == 1024 ? wq : (wq & 1)) * 256 + lane * 4;
    const int wgrp = woff / kChunkScales, wwithin = woff - wgrp * kChunkScales;
    wso = (uint32_t)min(gw0 + wgrp, g.gw - 1) * kChunkScales + wwithin;
  }
  const int64_t x_stage = (int64_t)g.gx * R::kChunkX, w_stage = (int64_t)g.gw * R::kChunkW;
  const int64_t xs_stage = (int64_t)g.gx * kChunkScales, ws_stage = (int64_t)g.gw * kChunkScales;
  const int xs_dst = R::kOffXs + xq * 256;
  const int ws_dst = R::kOffWs + (R::kStageScalesW == 1024 ? wq : (wq & 1)) * 256;
  const bool x_scale_wave = WV == 4 || wave < 4;  // 8 waves: which scale run this wave copies

  // copy number idx (0 .. kCopies-1) of this wave's share of stage ks into
  // ring slot `slot`: activation codes, weight codes, activation scales,
  // weight scales
  auto issue_one = [&](int idx, int ks, int slot) {
    uint8_t* base = lds + slot * R::kSlot;
    if (idx < R::kCX) {
      copy16_to_lds(g.x_codes + ks * x_stage + xo[idx], base + R::kOffX + (wave * R::kCX + idx) * 1024);
    } else if (idx < R::kCX + R::kCW) {
      const int i = idx - R::kCX;
      copy16_to_lds(g.w_codes + ks * w_stage + wo[i], base + R::kOffW + (wave * R::kCW + i) * 1024);
    } else if (idx == R::kCX + R::kCW && x_scale_wave) {
      copy4_to_lds(g.x_scales + ks * xs_stage + xso, base + xs_dst);
    } else {
      copy4_to_lds(g.w_scales + ks * ws_stage + wso, base + ws_dst);
    }
  };
  auto issue_range = [&](int ks, int slot, int first, int count) {
#pragma unroll
    for (int i = 0; i < count; ++i) issue_one(first + i, ks, slot);
  };

  // ---- per-lane LDS bases in ring slot 0; fragment f (32 rows) adds f chunks.
  // Half h of a chunk holds this lane's blocks 2h (sub-step 0) and 2h+1
  // (sub-step 1) in planes of 16 bytes per row (and, for the 6-bit types, of
  // 8 bytes per row).
  const int wn = wave % R::kWN, wm = wave / R::kWN;
  const int h = lane >> 5, j = lane & 31;
  const int wrow = feature_of_row<kLayout>(j);
  constexpr int kFW = R::kFW, kMP = R::kMfmaPhase;
  // chunk of the wave's first weight fragment and the chunk stride between
  // its fragments
  const int wchunk = kSwPair ? 4 * (wn / 2) + wn % 2 : wn * kFW;
  constexpr int kFragChunksW = kSwPair ? 2 : 1;
  const int w16 = R::kOffW + wchunk * R::kChunkW + h * R::kHalfW + wrow * 16;
  const int x16 = R::kOffX + wm * 4 * R::kChunkX + h * R::kHalfX + j * 16;
  const int w8 = R::kOffW + wchunk * R::kChunkW + h * R::kHalfW + wrow * 8;
  const int x8 = R::kOffX + wm * 4 * R::kChunkX + h * R::kHalfX + j * 8;
  const int wsc = R::kOffWs + wchunk * kChunkScales + wrow * 4 + 2 * h;
  const int xsc = R::kOffXs + wm * 4 * kChunkScales + j * 4 + 2 * h;

  v16f acc[kFW][4];
#pragma unroll
  for (int fn = 0; fn < kFW; ++fn)
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fn][fm][r] = 0.0f;

  // One sub-step operand of a 6-bit type is a 16-byte and an 8-byte LDS read
  // landing in adjacent registers (the MFMA reads 6 of the 8); of an 8-bit
  // type two 16-byte reads; of a 4-bit type one 16-byte read (the MFMA reads
  // 4 registers).  With 4- and 6-bit operands a lane's registers hold the 32
  // elements of its half's block; with 8-bit operands registers 0-3 of both
  // lane halves make the first 32-element block of the instruction's K = 64
  // (scaled by the byte of lanes 0-31) and registers 4-7 the second (scaled
  // by lanes 32-63), so in sub-step s lane half h holds bytes 16h..16h+15 of
  // blocks s and 2 + s, which the 8-bit layout's planes 2s and 2s + 1 store.
  // The 8-byte reads are volatile so they are not fused into one 16-byte read
  // whose halves would belong to different operands (that costs register
  // moves).
  typedef const volatile __attribute__((address_space(3))) u32x2 lds_u32x2_t;
  auto rd16 = [&](int off) { return *reinterpret_cast<const u32x4*>(lds + off); };
  auto rd8 = [&](int off) { return (u32x2)(*(lds_u32x2_t*)(lds + off)); };
  // operand of sub-step SUB for an operand of BITS-bit codes at lane bases b16 / b8
  auto op = [&](auto bits_tag, auto sub_tag, int b16, int b8) {
    constexpr int BITS = decltype(bits_tag)::value, SUB = decltype(sub_tag)::value;
    if constexpr (BITS == 6) {
      if constexpr (SUB == 0) {
        const u32x4 a = rd16(b16 + kPlaneA);
        const u32x2 c = rd8(b8 + kPlaneL);
        return v8i{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], 0, 0};
      } else {
        const u32x2 c = rd8(b8 + kPlaneH);
        const u32x4 a = rd16(b16 + kPlaneB);
        return v8i{(int)c[0], (int)c[1], (int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0};
      }
    } else if constexpr (BITS == 8) {
      const u32x4 a = rd16(b16 + (2 * SUB) * kPlaneStride16);
      const u32x4 c = rd16(b16 + (2 * SUB + 1) * kPlaneStride16);
      return v8i{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
    } else {
      const u32x4 a = rd16(b16 + SUB * kPlaneStride16);
      return v8i{(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
    }
  };
  using bw_t = std::integral_constant<int, R::kBW>;
  using bx_t = std::integral_constant<int, R::kBX>;
  constexpr int kDsW = R::kBW == 4 ? 1 : 2, kDsX = R::kBX == 4 ? 1 : 2;  // LDS reads per operand
  constexpr int kNF = kFW + 4;  // fragments per sub-step (and scale pairs per stage)
  struct Half {  // one sub-step's operands: kFW weight and 4 activation fragments
    v8i w[kFW], x[4];
  };
  struct Scales {  // scale byte pairs (blocks 2h, 2h+1) of the fragments
    int w[kFW], x[4];
  };
  // fragment i (0 .. kNF-1) of a sub-step, in the order w0, x0, w1, x1, ...,
  // then the activation fragments left over
  auto frag_is_w = [](int i) { return i < 2 * kFW && i % 2 == 0; };
  auto frag_index = [](int i) { return i < 2 * kFW ? i / 2 : i - kFW; };
  auto read_frag = [&](Half& r, int so, auto i_tag, auto sub_tag) {
    constexpr int I = decltype(i_tag)::value;
    constexpr int F = frag_index(I);
    if constexpr (frag_is_w(I))
      r.w[F] = op(bw_t{}, sub_tag, so + w16 + F * kFragChunksW * R::kChunkW,
                  so + w8 + F * kFragChunksW * R::kChunkW);
    else
      r.x[F] = op(bx_t{}, sub_tag, so + x16 + F * R::kChunkX, so + x8 + F * R::kChunkX);
  };
  auto read_half = [&](int sl, auto sub_tag) {
    const int so = sl * R::kSlot;
    Half r;
    static_for([&](auto i) { if constexpr (decltype(i)::value < kNF) read_frag(r, so, i, sub_tag); }, SeqN<kMP>{});
    return r;
  };
  auto scale_at = [&](int so, int base, int f) {
    return (int)*reinterpret_cast<const uint16_t*>(lds + so + base + f * kChunkScales);
  };
  // scale pair s (0 .. kNF-1): the weight fragments' first, then the activations'
  auto read_scale = [&](Scales& c, int so, auto s_tag) {
    constexpr int S = decltype(s_tag)::value;
    if constexpr (S < kFW)
      c.w[S] = scale_at(so, wsc, S * kFragChunksW);
    else
      c.x[S - kFW] = scale_at(so, xsc, S - kFW);
  };
  auto read_scales = [&](int sl) {
    const int so = sl * R::kSlot;
    Scales c;
    static_for([&](auto i) { if constexpr (decltype(i)::value < kNF) read_scale(c, so, i); }, SeqN<kMP>{});
    return c;
  };
  // MFMA i (0 .. kMP-1) of a sub-step: weight fragment i / 4 against activation fragment i % 4
  auto mfma = [&](const Half& r, const Scales& c, auto i_tag, auto sub_tag) {
    constexpr int I = decltype(i_tag)::value, S = decltype(sub_tag)::value;
    constexpr int FN = I / 4, FM = I % 4;
    acc[FN][FM] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(r.w[FN], r.x[FM], acc[FN][FM], WF, XF, S, c.w[FN],
                                                                 S, c.x[FM]);
  };
  // the MFMAs of one sub-step
  auto mfmas = [&](const Half& r, const Scales& c, auto sub_tag) {
    static_for([&](auto i) { mfma(r, c, i, sub_tag); }, SeqN<kMP>{});
  };
  using sub0 = std::integral_constant<int, 0>;
  using sub1 = std::integral_constant<int, 1>;
  // The steady-state phases, written in issue order (the LDS reads and the
  // copies into LDS keep their program order) and pinned for the scheduler
  // by sched_group_barrier: after MFMA i, the LDS reads of fragment i (i <
  // kNF) or, in phase 1, of the scale pairs scheduled after it, then the
  // copies scheduled after it.
  // Phase 1: sub-step 1 MFMAs, reads of the next stage's sub-step 0 operands
  // and scales, and the first kFirst copies of stage ks2 into slot slot2.
  auto phase1 = [&](const Half& r, const Scales& c, int ks2, int slot2, int nsl, Half& nr, Scales& ns, auto copy_tag) {
    constexpr bool kCopy = decltype(copy_tag)::value;
    const int so = nsl * R::kSlot;
    static_for(
        [&](auto i) {
          constexpr int I = decltype(i)::value;
          mfma(r, c, i, sub1{});
          if constexpr (I < kNF) read_frag(nr, so, i, sub0{});
          constexpr int nsr = scale_reads_after(I, kNF, kNF, kMP);
          if constexpr (nsr > 0) {
            constexpr int s0 = (I - kNF) * scales_per_mfma(kNF, kNF, kMP);
            static_for([&](auto k) {
              if constexpr (decltype(k)::value < nsr) read_scale(ns, so, std::integral_constant<int, s0 + decltype(k)::value>{});
            }, SeqN<kMP>{});
          }
          constexpr int n = kCopy ? copies_after(I, R::kFirst, 1, kMP) : 0;
          constexpr int c0 = first_copy_after(I, R::kFirst, 1, kMP);
#pragma unroll
          for (int k = 0; k < n; ++k) issue_one(c0 + k, ks2, slot2);
        },
        SeqN<kMP>{});
    static_for(
        [&](auto i) {
          constexpr int I = decltype(i)::value;
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          constexpr int ds = (I < kNF ? (frag_is_w(I) ? kDsW : kDsX) : 0) + scale_reads_after(I, kNF, kNF, kMP);
          if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds, 0);
          constexpr int n = kCopy ? copies_after(I, R::kFirst, 1, kMP) : 0;
          if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x020, n, 0);
        },
        SeqN<kMP>{});
  };
  // Phase 0: sub-step 0 MFMAs, reads of the same stage's sub-step 1
  // operands, and copies kFirst.. of stage ks2 into slot slot2.
  auto phase0 = [&](const Half& r, const Scales& c, int sl, Half& nr, int ks2, int slot2, auto copy_tag) {
    constexpr bool kCopy = decltype(copy_tag)::value;
    const int so = sl * R::kSlot;
    static_for(
        [&](auto i) {
          constexpr int I = decltype(i)::value;
          mfma(r, c, i, sub0{});
          if constexpr (I < kNF) read_frag(nr, so, i, sub1{});
          constexpr int n = kCopy ? copies_after(I, R::kSecond, 0, kMP) : 0;
          constexpr int c0 = first_copy_after(I, R::kSecond, 0, kMP);
#pragma unroll
          for (int k = 0; k < n; ++k) issue_one(R::kFirst + c0 + k, ks2, slot2);
        },
        SeqN<kMP>{});
    static_for(
        [&](auto i) {
          constexpr int I = decltype(i)::value;
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          constexpr int ds = I < kNF ? (frag_is_w(I) ? kDsW : kDsX) : 0;
          if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds, 0);
          constexpr int n = kCopy ? copies_after(I, R::kSecond, 0, kMP) : 0;
          if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x020, n, 0);
        },
        SeqN<kMP>{});
  };
  using copies = std::true_type;
  using no_copies = std::false_type;
  auto next_slot = [](int sl) { return sl + 1 == R::kSlots ? 0 : sl + 1; };

  // ---- main loop over the ring, with the operand registers double buffered
  // at half-stage granularity.  At the top of stage ks the lane holds stage
  // ks's sub-step 0 operands (ra) and scales (sc).  Phase 0: sub-step 0 MFMAs
  // while reading stage ks's sub-step 1 operands (rb) (and, with three slots,
  // issuing the second half of stage ks+2's copies).  Then wait until stage
  // ks+1 has landed (copies complete in order: with three slots at most stage
  // ks+2's copies may still be outstanding, with two none), and barrier: every
  // wave's part of stage ks+1 is visible and every wave is done reading slot
  // ks.  Phase 1: sub-step 1 MFMAs while reading stage ks+1's sub-step 0
  // operands and scales and issuing copies of stage ks+kSlots into slot ks.
  constexpr int kMidWait = R::kSlots == 3 ? R::kCopies : 0;
  if (nk > 0) issue_range(0, 0, 0, R::kCopies);
  if (nk > 1) issue_range(1, 1, 0, R::kCopies);
  if constexpr (R::kSlots == 3) {
    if (nk > 2) issue_range(2, 2, 0, R::kFirst);
    if (nk > 2)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(R::kCopies + R::kFirst));
    else if (nk > 1)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(R::kCopies));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  } else {
    if (nk > 1)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(R::kCopies));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  }
  __builtin_amdgcn_s_barrier();
  Half ra = read_half(0, sub0{});
  Scales sc = read_scales(0);
  int ks = 0, slot = 0;
  for (; ks + R::kSlots < nk; ++ks) {
    const int nsl = next_slot(slot);
    Half rb;
    phase0(ra, sc, slot, rb, ks + 2, next_slot(nsl), copies{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kMidWait));
    __builtin_amdgcn_s_barrier();
    Scales sn;
    phase1(rb, sc, ks + R::kSlots, slot, nsl, ra, sn, copies{});
    __builtin_amdgcn_sched_barrier(0);
    sc = sn;
    slot = nsl;
  }
  // The last kSlots stages, straight-line, with the steady state's phases:
  // only the copies that still exist (with three slots, the second half of
  // stage nk - 1's, in the first of them), and the wait for the next stage
  // tightened to every copy once no copy of a later stage is outstanding.
  // Sharing the phases keeps the steady state's register allocation: the
  // generic loop below spilled address registers in the 6- and 8-bit kernels,
  // and each reload waited for every copy in flight (fc1: 508 -> 480 us,
  // bit-identical).  4-bit operands keep the loop, which does not spill there
  // and measured 2.5 % faster with 8 waves.
  if (R::kBW != 4 && nk >= R::kSlots) {
    if constexpr (R::kSlots == 3) {
      const int nsl = next_slot(slot);
      Half rb;
      phase0(ra, sc, slot, rb, ks + 2, next_slot(nsl), copies{});
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(R::kCopies));
      __builtin_amdgcn_s_barrier();
      Scales sn;
      phase1(rb, sc, 0, 0, nsl, ra, sn, no_copies{});
      __builtin_amdgcn_sched_barrier(0);
      sc = sn;
      slot = nsl;
      ++ks;
    }
    {
      const int nsl = next_slot(slot);
      Half rb;
      phase0(ra, sc, slot, rb, 0, 0, no_copies{});
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
      __builtin_amdgcn_s_barrier();
      Scales sn;
      phase1(rb, sc, 0, 0, nsl, ra, sn, no_copies{});
      __builtin_amdgcn_sched_barrier(0);
      sc = sn;
      slot = nsl;
      ++ks;
    }
    {
      Half rb;
      phase0(ra, sc, slot, rb, 0, 0, no_copies{});
      __builtin_amdgcn_sched_barrier(0);
      mfmas(rb, sc, sub1{});
      ks = nk;
    }
  }
  for (; ks < nk; ++ks) {  // K shorter than the ring (and the 4-bit operands' tail)
    const int nsl = next_slot(slot);
    if constexpr (R::kSlots == 3) {
      if (ks + 2 < nk) issue_range(ks + 2, next_slot(nsl), R::kFirst, R::kSecond);
    }
    const Half rb = read_half(slot, sub1{});
    mfmas(ra, sc, sub0{});
    Scales sn = sc;
    if (ks + 1 < nk) {
      if (R::kSlots == 3 && ks + 2 < nk)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(R::kCopies));
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
  const int mw0 = m0 + wm * 128, nw0 = n0 + wn * (TN / R::kWN);
  // SwiGLU: the wave's weight fragments are its gate rows (the first kFW / 2)
  // and the up rows of the same features (the rest), output features
  // nw0/2 .. nw0/2 + 16 kFW - 1.
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
    // the swap, block scale and conversion: lane half h ends with the 24 code
    // bytes q and the scale byte of one whole block (va's for h = 0, vb's for h = 1)
    // A non-finite block comes back with scale byte 0xFF and its codes are
    // zeroed when it is stored (together with the layout padding).
    auto convert_pair = [&](const v16f& va, const v16f& vb, v6u& q, uint32_t& sbyte) {
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
      float amax = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = absmax2(amax, lo[r], hi[r]);
      const BlockScale sc = scale_from_f32_bits<OFMT>(__float_as_uint(amax));
      v16f ev, od;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ev[i] = lo[i];
        ev[8 + i] = hi[i];
        od[i] = lo[8 + i];
        od[8 + i] = hi[8 + i];
      }
      q = cvt_f32x2x16<OFMT>(ev, od, sc.scale);
      sbyte = sc.byte;
    };
    // block qb (0..3) of output stage `stage` for token row m of group gm:
    // even block: plane A (bytes 0..15) + plane L (16..23); odd block: plane
    // H (bytes 0..7) + plane B (8..23)
    auto store_block = [&](v6u q, uint32_t sbyte, int m, int gm, int stage, int qb) {
      const int nb = stage * 4 + qb;
      if (gm < g.gx && stage < n_stages) {
        const bool pad = m >= g.M || nb >= n_out / 32;  // layout padding: codes 0, scale 127
        if (pad || sbyte == 0xFFu) q = v6u{0, 0, 0, 0, 0, 0};  // padding or a non-finite block
        if (pad) sbyte = 127u;
        const bool odd = qb & 1;
        uint8_t* half =
            static_cast<uint8_t*>(g.out) + ((int64_t)stage * g.gx + gm) * kChunkCodes + (qb >> 1) * kHalfBytes;
        const u32x4 d16 = !odd ? u32x4{q[0], q[1], q[2], q[3]} : u32x4{q[2], q[3], q[4], q[5]};
        const u32x2 d8 = !odd ? u32x2{q[4], q[5]} : u32x2{q[0], q[1]};
        *reinterpret_cast<u32x4*>(half + (!odd ? kPlaneA : kPlaneB) + j * 16) = d16;
        *reinterpret_cast<u32x2*>(half + (!odd ? kPlaneL : kPlaneH) + j * 8) = d8;
        g.out_scales[((int64_t)stage * g.gx + gm) * kChunkScales + j * 4 + qb] = (uint8_t)sbyte;
      }
    };
    // two consecutive blocks 2pr, 2pr+1 of one token fragment (lane half h: block 2pr + h)
    auto emit_pair = [&](const v16f& va, const v16f& vb, int m, int gm, int stage, int pr) {
      v6u q;
      uint32_t sbyte;
      convert_pair(va, vb, q, sbyte);
      store_block(q, sbyte, m, gm, stage, 2 * pr + h);
    };
    if constexpr (kSwPair) {
      // SwiGLU with two fragments per wave: the wave's 32 output features
      // nw0/2 .. +31 are one block; pair token fragments fp and fp + 1 instead
      // (lane half h: the block of token fragment fp + h)
      const int ob = nw0 / 2;
      const int stage = ob / kTileStageK, qb = (ob % kTileStageK) / 32;
#pragma unroll
      for (int fp = 0; fp < 4; fp += 2) {
        v16f va, vb;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          va[r] = silu_f32(acc[0][fp][r]) * acc[1][fp][r];
          vb[r] = silu_f32(acc[0][fp + 1][r]) * acc[1][fp + 1][r];
        }
        v6u q;
        uint32_t sbyte;
        convert_pair(va, vb, q, sbyte);
        const int mrow0 = mw0 + (fp + h) * 32;
        store_block(q, sbyte, mrow0 + j, mrow0 / kTileGroupRows, stage, qb);
        // 128-feature tiles (64 output features, half a stage): the stage's
        // other 64 features have no tile when the output ends here, so write
        // their layout padding (block index past n_out / 32).  A 256-feature
        // tile covers its whole output stage, every block by its own wave.
        if (kSwNarrow && qb < 2 && n0 / 2 + 64 >= n_out)
          store_block(q, sbyte, mrow0 + j, mrow0 / kTileGroupRows, stage, qb + 2);
      }
      return;
    }
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
        // the wave's kFW fragments are kFW / 2 block pairs of output stage nw0 / 128
#pragma unroll
        for (int pr = 0; pr < kFW / 2; ++pr) {
          v16f va = acc[2 * pr][fm], vb = acc[2 * pr + 1][fm];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            va[r] = act(va[r]);
            vb[r] = act(vb[r]);
          }
          emit_pair(va, vb, m, gm, nw0 / kTileStageK, (nw0 % kTileStageK) / 64 + pr);
        }
      }
    }
    return;
  }
  constexpr int kOutFrags = kSwiglu ? kFW / 2 : kFW;
#pragma unroll
  for (int fn = 0; fn < kOutFrags; ++fn) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
      const int m = mw0 + fm * 32 + j;
      v16f v;
      if constexpr (kSwiglu) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = silu_f32(acc[fn][fm][r]) * acc[fn + kFW / 2][fm][r];
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

template <int WF, int XF, int EPI, int TN, int WV = 4>
void launch_epi(const GemmArgs& a, int out_kind, int out_fmt, dim3 grid, hipStream_t stream) {
  const dim3 block(64 * WV);
  if (out_kind == kOutF32)
    hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutF32, EPI, kFmtE2M3, TN, WV>), grid, block, 0, stream, a);
  else if (out_kind == kOutBf16)
    hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutBf16, EPI, kFmtE2M3, TN, WV>), grid, block, 0, stream, a);
  else if (out_fmt == kFmtE2M3)
    hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutMx, EPI, kFmtE2M3, TN, WV>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutMx, EPI, kFmtE3M2, TN, WV>), grid, block, 0, stream, a);
}

// The 6-bit pairs: every epilogue and output kind.
template <int WF, int XF>
hipError_t launch_variant(const GemmArgs& a, int epilogue, int out_kind, int out_fmt, hipStream_t stream,
                          std::true_type) {
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n));
  if (a.tile_n == 128) {
    if (a.waves != 4) return hipErrorInvalidValue;
    if (epilogue == kEpiGeluTanh)
      launch_epi<WF, XF, kEpiGeluTanh, 128>(a, out_kind, out_fmt, grid, stream);
    else if (epilogue == kEpiSwiglu)
      launch_epi<WF, XF, kEpiSwiglu, 128>(a, out_kind, out_fmt, grid, stream);
    else
      launch_epi<WF, XF, kEpiNone, 128>(a, out_kind, out_fmt, grid, stream);
    return hipGetLastError();
  }
  if (a.waves == 8) {
    if (epilogue == kEpiGeluTanh)
      launch_epi<WF, XF, kEpiGeluTanh, 256, 8>(a, out_kind, out_fmt, grid, stream);
    else if (epilogue == kEpiSwiglu)
      launch_epi<WF, XF, kEpiSwiglu, 256, 8>(a, out_kind, out_fmt, grid, stream);
    else
      launch_epi<WF, XF, kEpiNone, 256, 8>(a, out_kind, out_fmt, grid, stream);
    return hipGetLastError();
  }
  if (epilogue == kEpiGeluTanh)
    launch_epi<WF, XF, kEpiGeluTanh, 256>(a, out_kind, out_fmt, grid, stream);
  else if (epilogue == kEpiSwiglu)
    launch_epi<WF, XF, kEpiSwiglu, 256>(a, out_kind, out_fmt, grid, stream);
  else
    launch_epi<WF, XF, kEpiNone, 256>(a, out_kind, out_fmt, grid, stream);
  return hipGetLastError();
}

// The 4- and 8-bit operand formats: plain product, fp32 or bf16 output.
template <int WF, int XF>
hipError_t launch_variant(const GemmArgs& a, int epilogue, int out_kind, int, hipStream_t stream, std::false_type) {
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n));
  if (epilogue != kEpiNone || out_kind == kOutMx || a.tile_n != 256) return hipErrorInvalidValue;
  if (a.waves == 8) {
    const dim3 block(Ring<WF, XF, 256, 8>::kThreads);
    if (out_kind == kOutF32)
      hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutF32, kEpiNone, kFmtE2M3, 256, 8>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutBf16, kEpiNone, kFmtE2M3, 256, 8>), grid, block, 0, stream, a);
    return hipGetLastError();
  }
  const dim3 block(Ring<WF, XF>::kThreads);
  if (out_kind == kOutF32)
    hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutF32, kEpiNone, kFmtE2M3>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_kernel<WF, XF, kOutBf16, kEpiNone, kFmtE2M3>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// One translation unit per (weight, activation) format pair, so the variants
// build in parallel.
template <int WF, int XF>
hipError_t launch_gemm_formats(const GemmArgs& a, int epilogue, int out_kind, int out_fmt, hipStream_t stream) {
  return launch_variant<WF, XF>(a, epilogue, out_kind, out_fmt, stream,
                                std::integral_constant<bool, fmt_bits(WF) == 6 && fmt_bits(XF) == 6>{});
}

}  // namespace mxg
