// Skinny MX GEMM (M <= 16 tokens) for gfx950, split along K.
//
// The split-K idea is the one of the page "Creating Custom Kernels for the AMD
// MI300", section "Skinny GEMM Kernel": with few rows there are too few output
// tiles to occupy the GPU, so K is cut into S contiguous chunks computed
// concurrently.  Here the work is a pure stream of packed weights from HBM
// (0.78 bytes per weight), so the kernel is built for memory-level
// parallelism, not for the matrix cores:
//
//  * V_MFMA_SCALE_F32_16X16X128_F8F6F4 with the weights as the A operand
//    (16 feature rows) and the tokens as the B operand (16 columns, rows
//    >= M fed as zeros, so M = 8 costs no extra bytes).
//  * Inside a group of 4 consecutive MFMAs (512 K), lane group q of step s
//    handles K-block 4q + s.  Each lane therefore loads 96 contiguous bytes
//    (6 x 128-bit loads) and its 4 scale bytes as one dword; op_sel = s picks
//    the byte.
//  * Each wave streams 2 fragments (32 features) of its K-chunk with the next
//    group's loads in flight; there is no LDS and no barrier.
//  * fp32 partial sums go to a workspace [S, 16, N]; a second kernel adds the
//    S partials in the fixed order 0..S-1 and rounds once (deterministic).
#include "internal.h"
#include "mx_device.h"

namespace mxg {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kSkThreads = 256;
constexpr int kFragsPerWave = 2;                       // 16-feature fragments per wave
constexpr int kWaveFeatures = 16 * kFragsPerWave;      // 32
constexpr int kWgFeatures = 4 * kWaveFeatures;         // 128 features per workgroup
constexpr int kGroupK = 512;                           // K per group of 4 MFMAs
constexpr int kGroupBytes = 384;                       // packed bytes per row per group

struct Frag {
  u32x4 d[6];
  uint32_t s;
};

template <int WF, int XF>
__device__ __forceinline__ void mfma_group(v4f& acc, const Frag& w, const Frag& x) {
  // step s uses bytes [24 s, 24 s + 24) of the lane's 96 bytes: dwords 6s .. 6s+5
  const uint32_t* wd = reinterpret_cast<const uint32_t*>(w.d);
  const uint32_t* xd = reinterpret_cast<const uint32_t*>(x.d);
#define MXG_STEP(S)                                                                                             \
  {                                                                                                             \
    const v8i a = v8i{(int)wd[6 * S], (int)wd[6 * S + 1], (int)wd[6 * S + 2], (int)wd[6 * S + 3],           \
                      (int)wd[6 * S + 4], (int)wd[6 * S + 5], 0, 0};                                          \
    const v8i b = v8i{(int)xd[6 * S], (int)xd[6 * S + 1], (int)xd[6 * S + 2], (int)xd[6 * S + 3],           \
                      (int)xd[6 * S + 4], (int)xd[6 * S + 5], 0, 0};                                          \
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, WF, XF, S, (int)w.s, S, (int)x.s);       \
  }
  MXG_STEP(0)
  MXG_STEP(1)
  MXG_STEP(2)
  MXG_STEP(3)
#undef MXG_STEP
}

// grid: (ceil(N / 128), splits).  Each wave: 32 features x one K-chunk.
template <int WF, int XF>
__global__ __launch_bounds__(kSkThreads) void splitk_kernel(const SplitKArgs g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int split = blockIdx.y;
  const int kchunk = g.K / g.splits;
  const int ngroups = kchunk / kGroupK;
  const int64_t rowbytes = (int64_t)g.K * 3 / 4;
  const int kblocks = g.K / 32;
  const int nbase = blockIdx.x * kWgFeatures + wave * kWaveFeatures;

  // this lane's rows: token r16 of the activations, feature nbase + 16f + r16 of the weights
  const bool xvalid = r16 < g.M;
  const int64_t kbyte0 = (int64_t)split * kchunk * 3 / 4 + 96 * q;
  const int kblk0 = split * (kchunk / 32) + 4 * q;
  const uint8_t* xp = g.x_codes + (int64_t)(xvalid ? r16 : 0) * rowbytes + kbyte0;
  const uint8_t* xs = g.x_scales + (int64_t)(xvalid ? r16 : 0) * kblocks + kblk0;
  const uint8_t* wp[kFragsPerWave];
  const uint8_t* wsp[kFragsPerWave];
#pragma unroll
  for (int f = 0; f < kFragsPerWave; ++f) {
    const int n = min(nbase + 16 * f + r16, g.N - 1);
    wp[f] = g.w_codes + (int64_t)n * rowbytes + kbyte0;
    wsp[f] = g.w_scales + (int64_t)n * kblocks + kblk0;
  }

  auto load = [&](int grp, Frag& x, Frag (&w)[kFragsPerWave]) {
    const int64_t bo = (int64_t)grp * kGroupBytes;
    const int so = grp * 16;
#pragma unroll
    for (int f = 0; f < kFragsPerWave; ++f) {
#pragma unroll
      for (int i = 0; i < 6; ++i) w[f].d[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp[f] + bo) + i);
      w[f].s = *reinterpret_cast<const uint32_t*>(wsp[f] + so);
    }
    if (xvalid) {
#pragma unroll
      for (int i = 0; i < 6; ++i) x.d[i] = *(reinterpret_cast<const u32x4*>(xp + bo) + i);
      x.s = *reinterpret_cast<const uint32_t*>(xs + so);
    } else {
#pragma unroll
      for (int i = 0; i < 6; ++i) x.d[i] = u32x4{0u, 0u, 0u, 0u};
      x.s = 0x7f7f7f7fu;
    }
  };

  v4f acc[kFragsPerWave];
#pragma unroll
  for (int f = 0; f < kFragsPerWave; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};

  Frag xa, xb, wa[kFragsPerWave], wb[kFragsPerWave];
  if (ngroups > 0) load(0, xa, wa);
  for (int grp = 0; grp < ngroups; grp += 2) {
    if (grp + 1 < ngroups) load(grp + 1, xb, wb);
#pragma unroll
    for (int f = 0; f < kFragsPerWave; ++f) mfma_group<WF, XF>(acc[f], wa[f], xa);
    if (grp + 1 < ngroups) {
      if (grp + 2 < ngroups) load(grp + 2, xa, wa);
#pragma unroll
      for (int f = 0; f < kFragsPerWave; ++f) mfma_group<WF, XF>(acc[f], wb[f], xb);
    }
  }

  // lane holds features nbase + 16f + 4q + (0..3) for token r16
  if (r16 < g.M) {
    float* part = g.partial + ((int64_t)split * 16 + r16) * g.N;
#pragma unroll
    for (int f = 0; f < kFragsPerWave; ++f) {
      const int n = nbase + 16 * f + 4 * q;
      if (n + 4 <= g.N && (g.N & 3) == 0) {
        *reinterpret_cast<v4f*>(part + n) = acc[f];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < g.N) part[n + i] = acc[f][i];
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
  const dim3 grid((unsigned)((a.N + kWgFeatures - 1) / kWgFeatures), (unsigned)a.splits), block(kSkThreads);
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
