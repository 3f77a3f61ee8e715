// Skinny MX GEMM (M <= 16 tokens) for gfx950, split along K.
//
// The split-K idea is the one of the page "Creating Custom Kernels for the AMD
// MI300", section "Skinny GEMM Kernel": with few rows there are too few output
// tiles to occupy the GPU, so K is cut into S contiguous chunks computed
// concurrently and their partial sums are reduced.  Here the work is a pure
// stream of packed weights from HBM (0.78 bytes per weight), so the kernel is
// built for memory-level parallelism, not for the matrix cores:
//
//  * One workgroup per pair of 32-feature weight groups, 4 waves.  Wave w
//    streams the K-chunks w*spw .. w*spw+spw-1 (spw = ceil(S/4)) of both
//    groups, stage after stage, with kWindow stages of loads in flight across
//    chunk boundaries.  Each stage's activation operand is loaded once and
//    used by the MFMAs of both groups: the activations are the same few
//    hundred KB for every workgroup and come from L2, so sharing them halves
//    those load instructions per weight byte (they measured a fifth of the
//    kernel's time with one group per wave).  208 workgroups of 4 waves for
//    N = 13312 fit the GPU in one round.
//  * Both operands are in the tiled MX layout.  Per 128-element stage each
//    lane loads its row's entries of the four planes of half h (16 + 8 + 8 +
//    16 bytes), so every load instruction reads contiguous runs of 512 or 256
//    bytes.  The weights are read once (non-temporal).
//  * V_MFMA_SCALE_F32_32X32X64_F8F6F4 with the weights as the A operand and
//    the tokens as the B operand; token rows 16..31 are layout padding (zero
//    codes), so M = 8 or 16 costs no extra weight bytes and no branches.
//  * The scale bytes a wave needs for all of its stages (both groups' weight
//    scales and the tokens' activation scales, 320 B per stage) are loaded
//    with a handful of 16-byte loads ahead of the first stages and kept in
//    the wave's own LDS slice, then read per stage from LDS.  That takes
//    three small loads per stage out of the in-order memory queue the weight
//    stream uses.
//  * The window only works if each MFMA waits for its own stage's loads and
//    not for all of them (vmcnt counts loads in issue order).  The compiler
//    inserts those waits; it can count exactly only when: a slot is consumed
//    in place before it is refilled (a copy of a register with a load
//    pending waits for every load), the per-wave bounds are uniform values,
//    every refill is unconditional (past the last stage it reads one line,
//    never used), and no direct global-to-LDS copy is pending (those make
//    every later LDS read wait for all loads).  The LDS-scale path meets all
//    four: every wave streams a multiple of kWindow stages, at most
//    kLdsStages.  Other shapes take the per-stage-scale path with
//    conditional refills.
//  * When a chunk ends, its fp32 partials go to LDS; after one barrier the
//    workgroup adds the S partials in the fixed order 0 .. S-1 (deterministic)
//    and rounds once into the output.  No partials touch HBM and no second
//    kernel is launched.
#include "grid_limits.h"
#include "internal.h"
#include "mx_device.h"

namespace mxg {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kSkWaves = 4;  // 32 stages per wave at K = 16384, S = 16: 8 waves of 16 stages
                              // spend a larger share of each stream filling and draining the window
constexpr int kSkThreads = 64 * kSkWaves;
constexpr int kSkGroups = 2;  // 32-feature weight groups per workgroup (and per wave)
constexpr int kWindow = 4;    // stages of loads in flight per wave
constexpr int kLdsStages = 32;  // stages per wave whose scales fit the wave's LDS slice
constexpr int kRecW = 2 * kChunkScales;  // per stage: both groups' weight scales (2 x 128 B)
constexpr int kRecX = kChunkScales / 2;  // per stage: token rows 0..15's activation scales
static_assert(kLdsStages % 16 == 0, "scale records load 4 (weights) and 16 (activations) stages per load");

// One operand pair of a stage as loaded: the lane's entries of planes A, L,
// H and B of half h (block 2h = A + L, block 2h+1 = H + B).  The window keeps
// these 12 dwords; the MFMA operands are assembled only at use.
struct Pieces {
  u32x4 a, b;
  u32x2 l, hh;
};

struct StageOps {
  Pieces w0, w1, x;  // the two weight groups' pieces and the activations'
  int ws0, ws1, xs;  // scale pairs (bytes 2h, 2h+1 of the lane's row)
};

template <bool NT>
__device__ __forceinline__ Pieces load_pieces(const uint8_t* half, int j) {
  const u32x4* pa = reinterpret_cast<const u32x4*>(half + kPlaneA + j * 16);
  const u32x2* pl = reinterpret_cast<const u32x2*>(half + kPlaneL + j * 8);
  const u32x2* ph = reinterpret_cast<const u32x2*>(half + kPlaneH + j * 8);
  const u32x4* pb = reinterpret_cast<const u32x4*>(half + kPlaneB + j * 16);
  Pieces p;
  if constexpr (NT) {
    p.a = __builtin_nontemporal_load(pa);
    p.l = __builtin_nontemporal_load(pl);
    p.hh = __builtin_nontemporal_load(ph);
    p.b = __builtin_nontemporal_load(pb);
  } else {
    p.a = *pa;
    p.l = *pl;
    p.hh = *ph;
    p.b = *pb;
  }
  return p;
}

__device__ __forceinline__ v8i op0(const Pieces& p) {
  return v8i{(int)p.a[0], (int)p.a[1], (int)p.a[2], (int)p.a[3], (int)p.l[0], (int)p.l[1], 0, 0};
}
__device__ __forceinline__ v8i op1(const Pieces& p) {
  return v8i{(int)p.hh[0], (int)p.hh[1], (int)p.b[0], (int)p.b[1], (int)p.b[2], (int)p.b[3], 0, 0};
}

// grid: one workgroup per pair of 32-feature groups.
// LDS_SCALES: every wave streams at most kLdsStages stages.
template <int WF, int XF, int OUT, bool LDS_SCALES>
__global__ __launch_bounds__(kSkThreads) void splitk_kernel(const SplitKArgs g) {
  // partial sums [split][token][feature], tokens 0..15, features of both groups.
  // Rows are padded by 4 floats: the 16 token lanes of a half-wave store 16
  // bytes each at the same feature offset, and with 256-byte rows they would
  // all land on the same four banks; 272-byte rows put them on 64 distinct banks.
  __shared__ __attribute__((aligned(16))) float part[kMaxSplits][16][32 * kSkGroups + 4];
  // per wave: the scale bytes of its stages, in stage order
  __shared__ __attribute__((aligned(16))) uint8_t scw[LDS_SCALES ? kSkWaves : 1][LDS_SCALES ? kLdsStages : 1][kRecW];
  __shared__ __attribute__((aligned(16))) uint8_t scx[LDS_SCALES ? kSkWaves : 1][LDS_SCALES ? kLdsStages : 1][kRecX];
  // the wave index as a uniform value: every per-wave bound and refill
  // condition below is then scalar, not an exec-masked branch
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, j = lane & 31;
  const int grp = blockIdx.x * kSkGroups;                 // first of the workgroup's groups
  const bool has1 = grp + 1 < g.gw;                      // the second group exists
  const int sps = g.K / kTileStageK / g.splits;          // stages per chunk
  const int spw = (g.splits + kSkWaves - 1) / kSkWaves;  // chunks per wave
  const int c0 = wave * spw;
  const int c1 = min(g.splits, c0 + spw);
  const int nst = c1 > c0 ? (c1 - c0) * sps : 0;         // stages this wave streams
  const int nc = c1 > c0 ? c1 - c0 : 0;                  // chunks of this wave
  // Every workgroup walks its chunks in a rotated order and each chunk's
  // stages from a rotated start, so that the workgroups, which all read the
  // same activations, spread their requests over many lines instead of
  // hammering the same few at the same time.  The order is fixed per pair of
  // groups (deterministic); the chunks' partials still meet in order 0 .. S-1.
  const int r0 = sps > 0 ? blockIdx.x % sps : 0;
  const int q0 = nc > 0 ? (blockIdx.x / max(sps, 1)) % nc : 0;
  const int lane_off = h * kHalfBytes;
  const int scale_off = j * 4 + 2 * h;
  const uint8_t* wc = g.w_codes + (int64_t)grp * kChunkCodes + lane_off;
  const uint8_t* ws = g.w_scales + (int64_t)grp * kChunkScales + scale_off;
  const uint8_t* xc = g.x_codes + lane_off;  // activations: one 32-row group
  const int64_t w_step = (int64_t)g.gw * kChunkCodes, ws_step = (int64_t)g.gw * kChunkScales;
  const bool token = j < 16;  // rows 16..31 of the activation group are zero padding

  // load cursor: chunk position cl (0 .. nc-1) and stage position tl (0 .. sps-1)
  int cl = 0, tl = 0;
  auto next_stage = [&]() {
    int c = cl + q0;
    c = c >= nc ? c - nc : c;
    int t = tl + r0;
    t = t >= sps ? t - sps : t;
    if (++tl == sps) {
      tl = 0;
      ++cl;
    }
    return (c0 + c) * sps + t;
  };
  const int s_first = c0 * sps;  // the wave's stages are s_first .. s_first + nst - 1
  // Loads are branch-free, so that the compiler can count the window's
  // loads exactly and wait for one stage at a time: padding lanes 16..31
  // re-read token rows 0..15 (the same lines, no extra requests) and a
  // missing second group re-reads the first; neither result is ever stored.
  const int jx = j & 15;
  const int64_t w1_off = has1 ? kChunkCodes : 0;
  const int64_t ws1_off = has1 ? kChunkScales : 0;
  const int xs_off = jx * 4 + 2 * h;
  auto load_codes = [&](int st, StageOps& o) {
    o.w0 = load_pieces<true>(wc + st * w_step, j);
    o.w1 = load_pieces<true>(wc + st * w_step + w1_off, j);
    o.x = load_pieces<false>(xc + (int64_t)st * kChunkCodes, jx);
  };
  auto load_scales_global = [&](int st, StageOps& o) {
    o.ws0 = *reinterpret_cast<const uint16_t*>(ws + st * ws_step);
    o.ws1 = *reinterpret_cast<const uint16_t*>(ws + st * ws_step + ws1_off);
    o.xs = *reinterpret_cast<const uint16_t*>(g.x_scales + (int64_t)st * kChunkScales + xs_off);
  };
  auto load_scales = [&](int st, StageOps& o) {
    if constexpr (LDS_SCALES) {
      const uint8_t* r = &scw[wave][st - s_first][scale_off];
      o.ws0 = *reinterpret_cast<const uint16_t*>(r);
      o.ws1 = *reinterpret_cast<const uint16_t*>(r + kChunkScales);
      o.xs = *reinterpret_cast<const uint16_t*>(&scx[wave][st - s_first][xs_off]);
    } else {
      load_scales_global(st, o);
    }
  };
  // LDS path refill, unconditional so that the compiler counts the loads in
  // flight exactly: past the wave's last stage (more == false) every lane
  // reads the same few lines at the start of the weights; never consumed.
  auto refill = [&](int st, bool more, StageOps& o) {
    const uint8_t* w = more ? wc + st * w_step : g.w_codes;
    const uint8_t* x = more ? xc + (int64_t)st * kChunkCodes : g.w_codes;
    const int jw = more ? j : 0, jt = more ? jx : 0;
    o.w0 = load_pieces<true>(w, jw);
    o.w1 = load_pieces<true>(more ? w + w1_off : w, jw);
    o.x = load_pieces<false>(x, jt);
    load_scales(more ? st : s_first, o);
  };
  auto load = [&](int st) {
    StageOps o;
    load_codes(st, o);
    load_scales(st, o);
    return o;
  };

  v16f acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.0f;
  StageOps win[kWindow];
  if constexpr (LDS_SCALES) {
    if (nst > 0) {  // then nst >= kWindow (launch condition)
      // The scale bytes of the wave's stages are loaded first (weight scales
      // 16 lanes x 16 B per stage, 4 stages per load, a missing second group
      // repeating the first; activation scales 4 lanes x 16 B per stage, 16
      // stages per load; lanes past the wave's last stage repeat it), then
      // the window's code loads, then the scales are written to the wave's
      // LDS slice: the wait for them is not a wait for the window.
      const uint8_t* wsb = g.w_scales + (int64_t)grp * kChunkScales + (has1 ? lane & 15 : lane & 7) * 16;
      u32x4 rw[kLdsStages / 4];
#pragma unroll
      for (int r = 0; r < kLdsStages / 4; ++r)
        rw[r] = *reinterpret_cast<const u32x4*>(wsb + (int64_t)(s_first + min(4 * r + (lane >> 4), nst - 1)) * ws_step);
      u32x4 rx[kLdsStages / 16];
#pragma unroll
      for (int r = 0; r < kLdsStages / 16; ++r)
        rx[r] = *reinterpret_cast<const u32x4*>(
            g.x_scales + (int64_t)(s_first + min(16 * r + (lane >> 2), nst - 1)) * kChunkScales + (lane & 3) * 16);
      int wst[kWindow];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kWindow; ++k) {
        wst[k] = next_stage();
        load_codes(wst[k], win[k]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < kLdsStages / 4; ++r)
        *reinterpret_cast<u32x4*>(&scw[wave][4 * r + (lane >> 4)][(lane & 15) * 16]) = rw[r];
#pragma unroll
      for (int r = 0; r < kLdsStages / 16; ++r)
        *reinterpret_cast<u32x4*>(&scx[wave][16 * r + (lane >> 2)][(lane & 3) * 16]) = rx[r];
#pragma unroll
      for (int k = 0; k < kWindow; ++k) load_scales(wst[k], win[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kWindow; ++k)
      if (k < nst) win[k] = load(next_stage());
  }
  int cc = 0, left = sps;  // chunk position being accumulated, its stages still to come
  for (int i = 0; i < nst; i += kWindow) {
#pragma unroll
    for (int k = 0; k < kWindow; ++k) {
      // LDS path: nst is a multiple of kWindow (launch condition)
      if (LDS_SCALES || i + k < nst) {
        // consume the slot in place, then refill it: the refill can reuse
        // the slot's registers, so the window rotates without copies (a copy
        // of a register with a load pending would wait for every load)
        const StageOps& o = win[k];
        const v8i x0 = op0(o.x), x1 = op1(o.x);
        acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op0(o.w0), x0, acc0, WF, XF, 0, o.ws0, 0, o.xs);
        acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op0(o.w1), x0, acc1, WF, XF, 0, o.ws1, 0, o.xs);
        acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op1(o.w0), x1, acc0, WF, XF, 1, o.ws0, 1, o.xs);
        acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op1(o.w1), x1, acc1, WF, XF, 1, o.ws1, 1, o.xs);
        if (--left == 0) {
          int chunk = cc + q0;
          chunk = c0 + (chunk >= nc ? chunk - nc : chunk);
          // lane (h, j) holds, for token j, features 8a + 4h + b in register 4a + b
          if (token) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              *reinterpret_cast<v4f*>(&part[chunk][j][8 * a + 4 * h]) =
                  v4f{acc0[4 * a], acc0[4 * a + 1], acc0[4 * a + 2], acc0[4 * a + 3]};
              *reinterpret_cast<v4f*>(&part[chunk][j][32 + 8 * a + 4 * h]) =
                  v4f{acc1[4 * a], acc1[4 * a + 1], acc1[4 * a + 2], acc1[4 * a + 3]};
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.0f;
          ++cc;
          left = sps;
        }
        if constexpr (LDS_SCALES) {
          const bool more = i + k + kWindow < nst;
          refill(next_stage(), more, win[k]);  // the cursor may run past the end: unused then
        } else if (i + k + kWindow < nst) {
          win[k] = load(next_stage());
        }
      }
    }
  }
  __syncthreads();

  // out[m, n] = round(sum_{s=0}^{S-1} part[s][m][n - 32 grp]), in that order
  const bool empty = sps == 0;  // K == 0
  for (int t = threadIdx.x; t < g.M * 32 * kSkGroups; t += kSkThreads) {
    const int m = t / (32 * kSkGroups), f = t % (32 * kSkGroups), n = grp * 32 + f;
    float sum = 0.0f;
    if (!empty)
      for (int s = 0; s < g.splits; ++s) sum += part[s][m][f];
    if (n < g.N) {
      if constexpr (OUT == kOutBf16) {
        const __bf16 b = (__bf16)sum;
        __builtin_memcpy(static_cast<uint16_t*>(g.out) + (int64_t)m * g.ldo + n, &b, 2);
      } else {
        static_cast<float*>(g.out)[(int64_t)m * g.ldo + n] = sum;
      }
    }
  }
}

template <int OUT, bool LDS_SCALES>
hipError_t launch_fmt(const SplitKArgs& a, int x_fmt, int w_fmt, hipStream_t stream) {
  const dim3 grid((unsigned)(splitk_grid_items(a.N) / kSkThreads)), block(kSkThreads);
  if (w_fmt == kFmtE2M3 && x_fmt == kFmtE2M3)
    hipLaunchKernelGGL((splitk_kernel<kFmtE2M3, kFmtE2M3, OUT, LDS_SCALES>), grid, block, 0, stream, a);
  else if (w_fmt == kFmtE3M2 && x_fmt == kFmtE2M3)
    hipLaunchKernelGGL((splitk_kernel<kFmtE3M2, kFmtE2M3, OUT, LDS_SCALES>), grid, block, 0, stream, a);
  else if (w_fmt == kFmtE2M3 && x_fmt == kFmtE3M2)
    hipLaunchKernelGGL((splitk_kernel<kFmtE2M3, kFmtE3M2, OUT, LDS_SCALES>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int OUT>
hipError_t launch_out(const SplitKArgs& a, int x_fmt, int w_fmt, hipStream_t stream) {
  // A wave streams 0 or 1 .. ceil(S / waves) chunks of K / 128 / S stages.
  // The LDS scale path needs every streaming wave to fill the window and to
  // fit its records in its slice.
  const int64_t sps = a.K / kTileStageK / a.splits;
  const bool lds = sps > 0 && sps % kWindow == 0 && ceil_div(a.splits, kSkWaves) * sps <= kLdsStages;
  return lds ? launch_fmt<OUT, true>(a, x_fmt, w_fmt, stream) : launch_fmt<OUT, false>(a, x_fmt, w_fmt, stream);
}

}  // namespace

// one workgroup per kSkGroups 32-feature weight groups
int64_t splitk_grid_items(int64_t n) { return ceil_div(ceil_div(n, kTileGroupRows), kSkGroups) * kSkThreads; }

hipError_t launch_gemm_splitk(const SplitKArgs& a, int x_fmt, int w_fmt, int out_kind, hipStream_t stream) {
  if (a.splits < 1 || a.splits > kMaxSplits || a.M > 16) return hipErrorInvalidValue;
  if (splitk_grid_items(a.N) > kMaxGridItems) return hipErrorInvalidConfiguration;
  return out_kind == kOutBf16 ? launch_out<kOutBf16>(a, x_fmt, w_fmt, stream)
                              : launch_out<kOutF32>(a, x_fmt, w_fmt, stream);
}

}  // namespace mxg
