// Skinny MX GEMM (M <= 16 tokens) for gfx950, split along K.
//
// The split-K idea is the one of the page "Creating Custom Kernels for the AMD
// MI300", section "Skinny GEMM Kernel": with few rows there are too few output
// tiles to occupy the GPU, so K is cut into S contiguous chunks computed
// concurrently.  Here the work is a pure stream of packed weights from HBM
// (0.78 bytes per weight), so the kernel is built for memory-level
// parallelism, not for the matrix cores:
//
//  * Both operands are in the tiled MX layout.  A wave owns one 32-feature
//    group of the weights and one K-chunk; per 128-element stage each lane
//    loads its row's entries of the four planes of half h (16 + 8 + 8 + 16
//    bytes), so every load instruction reads two contiguous runs of 512 or
//    256 bytes.
//  * V_MFMA_SCALE_F32_32X32X64_F8F6F4 with the weights as the A operand and
//    the tokens as the B operand; token rows 16..31 are layout padding (zero
//    codes), so M = 8 or 16 costs no extra weight bytes and no branches.
//  * A window of kWindow stages of loads stays in flight per wave (no LDS, no
//    barrier); the activations (a few hundred KB) come from L2.
//  * fp32 partial sums go to a workspace [S, 16, N]; a second kernel adds the
//    S partials in the fixed order 0..S-1 and rounds once (deterministic).
#include "internal.h"
#include "mx_device.h"

namespace mxg {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kSkThreads = 256;
constexpr int kWgGroups = 4;          // 32-feature groups per workgroup (one per wave)
constexpr int kWindow = 4;            // stages of loads in flight per wave

struct StageOps {
  v8i w0, w1, x0, x1;  // sub-step 0 / 1 operands
  int ws, xs;          // scale pairs (bytes 2h, 2h+1 of the lane's row)
};

// The two sub-step operands of lane (h, j) from the planes of half h of a
// chunk: block 2h = plane A + plane L, block 2h+1 = plane H + plane B.
template <bool NT>
__device__ __forceinline__ void load_ops(const uint8_t* half, int j, v8i& s0, v8i& s1) {
  const u32x4* pa = reinterpret_cast<const u32x4*>(half + kPlaneA + j * 16);
  const u32x2* pl = reinterpret_cast<const u32x2*>(half + kPlaneL + j * 8);
  const u32x2* ph = reinterpret_cast<const u32x2*>(half + kPlaneH + j * 8);
  const u32x4* pb = reinterpret_cast<const u32x4*>(half + kPlaneB + j * 16);
  u32x4 a, b;
  u32x2 l, hh;
  if constexpr (NT) {
    a = __builtin_nontemporal_load(pa);
    l = __builtin_nontemporal_load(pl);
    hh = __builtin_nontemporal_load(ph);
    b = __builtin_nontemporal_load(pb);
  } else {
    a = *pa;
    l = *pl;
    hh = *ph;
    b = *pb;
  }
  s0 = v8i{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)l[0], (int)l[1], 0, 0};
  s1 = v8i{(int)hh[0], (int)hh[1], (int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0};
}

// grid: (ceil(N / 128), splits).  Wave w: weight group blockIdx.x * 4 + w, K-chunk blockIdx.y.
template <int WF, int XF>
__global__ __launch_bounds__(kSkThreads) void splitk_kernel(const SplitKArgs g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, j = lane & 31;
  const int grp = blockIdx.x * kWgGroups + wave;
  if (grp >= g.gw) return;  // whole wave; the kernel has no barriers
  const int split = blockIdx.y;
  const int sps = g.K / kTileStageK / g.splits;  // stages per split
  const int s0 = split * sps;
  const int lane_off = h * kHalfBytes;
  const int scale_off = j * 4 + 2 * h;
  const uint8_t* wc = g.w_codes + ((int64_t)s0 * g.gw + grp) * kChunkCodes + lane_off;
  const uint8_t* ws = g.w_scales + ((int64_t)s0 * g.gw + grp) * kChunkScales + scale_off;
  const uint8_t* xc = g.x_codes + (int64_t)s0 * kChunkCodes + lane_off;  // activations: one 32-row group
  const uint8_t* xs = g.x_scales + (int64_t)s0 * kChunkScales + scale_off;
  const int64_t w_step = (int64_t)g.gw * kChunkCodes, ws_step = (int64_t)g.gw * kChunkScales;

  auto load = [&](int i) {
    StageOps o;
    load_ops<true>(wc + i * w_step, j, o.w0, o.w1);
    load_ops<false>(xc + (int64_t)i * kChunkCodes, j, o.x0, o.x1);
    o.ws = *reinterpret_cast<const uint16_t*>(ws + i * ws_step);
    o.xs = *reinterpret_cast<const uint16_t*>(xs + (int64_t)i * kChunkScales);
    return o;
  };

  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  StageOps win[kWindow];
#pragma unroll
  for (int i = 0; i < kWindow; ++i)
    if (i < sps) win[i] = load(i);
  for (int i = 0; i < sps; i += kWindow) {
#pragma unroll
    for (int k = 0; k < kWindow; ++k) {
      if (i + k < sps) {
        const StageOps o = win[k];
        if (i + k + kWindow < sps) win[k] = load(i + k + kWindow);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.w0, o.x0, acc, WF, XF, 0, o.ws, 0, o.xs);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.w1, o.x1, acc, WF, XF, 1, o.ws, 1, o.xs);
      }
    }
  }

  // lane (h, j) holds, for token j, features grp * 32 + 8a + 4h + b in register 4a + b
  if (j < g.M) {
    float* part = g.partial + ((int64_t)split * 16 + j) * g.N;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int n = grp * 32 + 8 * a + 4 * h;
      const v4f v = v4f{acc[4 * a], acc[4 * a + 1], acc[4 * a + 2], acc[4 * a + 3]};
      if (n + 4 <= g.N && (g.N & 3) == 0) {
        *reinterpret_cast<v4f*>(part + n) = v;
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (n + b < g.N) part[n + b] = v[b];
      }
    }
  }
}

// out[m, n] = round(sum_{s=0}^{S-1} partial[s, m, n]), summed in that order.
template <int OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const SplitKArgs g) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int nq = (g.N + 3) / 4;
  if (t >= (int64_t)g.M * nq) return;
  const int m = (int)(t / nq);
  const int n = (int)(t - (int64_t)m * nq) * 4;
  const bool vec = (g.N & 3) == 0;
  v4f s = v4f{0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < g.splits; ++sp) {
    const float* p = g.partial + ((int64_t)sp * 16 + m) * g.N + n;
    if (vec) {
      s += *reinterpret_cast<const v4f*>(p);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n + i < g.N) s[i] += p[i];
    }
  }
  if constexpr (OUT == kOutBf16) {
    uint16_t* o = static_cast<uint16_t*>(g.out) + (int64_t)m * g.ldo + n;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (n + i < g.N) {
        const __bf16 b = (__bf16)s[i];
        __builtin_memcpy(o + i, &b, 2);
      }
  } else {
    float* o = static_cast<float*>(g.out) + (int64_t)m * g.ldo + n;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (n + i < g.N) o[i] = s[i];
  }
}

}  // namespace

hipError_t launch_gemm_splitk(const SplitKArgs& a, int x_fmt, int w_fmt, int out_kind, hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(a.gw, kWgGroups), (unsigned)a.splits), block(kSkThreads);
  if (w_fmt == kFmtE2M3 && x_fmt == kFmtE2M3)
    hipLaunchKernelGGL((splitk_kernel<kFmtE2M3, kFmtE2M3>), grid, block, 0, stream, a);
  else if (w_fmt == kFmtE3M2 && x_fmt == kFmtE2M3)
    hipLaunchKernelGGL((splitk_kernel<kFmtE3M2, kFmtE2M3>), grid, block, 0, stream, a);
  else if (w_fmt == kFmtE2M3 && x_fmt == kFmtE3M2)
    hipLaunchKernelGGL((splitk_kernel<kFmtE2M3, kFmtE3M2>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = (int64_t)a.M * ((a.N + 3) / 4);
  const dim3 rgrid((unsigned)((threads + 255) / 256));
  if (out_kind == kOutBf16)
    hipLaunchKernelGGL(splitk_reduce_kernel<kOutBf16>, rgrid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<kOutF32>, rgrid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mxg
