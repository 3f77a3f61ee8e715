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

// One 16-row fragment over one 512-K group: the four MFMA operands (step s
// uses the lane's bytes [24 s, 24 s + 24)) and the lane's 4 scale bytes.
struct Ops {
  v8i s0, s1, s2, s3;
  uint32_t sc;
};

__device__ __forceinline__ Ops ops_from(const u32x4 d0, const u32x4 d1, const u32x4 d2, const u32x4 d3,
                                       const u32x4 d4, const u32x4 d5, uint32_t sc) {
  Ops o;
  o.s0 = v8i{(int)d0[0], (int)d0[1], (int)d0[2], (int)d0[3], (int)d1[0], (int)d1[1], 0, 0};
  o.s1 = v8i{(int)d1[2], (int)d1[3], (int)d2[0], (int)d2[1], (int)d2[2], (int)d2[3], 0, 0};
  o.s2 = v8i{(int)d3[0], (int)d3[1], (int)d3[2], (int)d3[3], (int)d4[0], (int)d4[1], 0, 0};
  o.s3 = v8i{(int)d4[2], (int)d4[3], (int)d5[0], (int)d5[1], (int)d5[2], (int)d5[3], 0, 0};
  o.sc = sc;
  return o;
}

// Streamed weights: non-temporal 128-bit loads (each byte is read once).
__device__ __forceinline__ Ops load_w(const uint8_t* p, const uint8_t* sp) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  return ops_from(__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1), __builtin_nontemporal_load(q + 2),
                  __builtin_nontemporal_load(q + 3), __builtin_nontemporal_load(q + 4),
                  __builtin_nontemporal_load(q + 5), *reinterpret_cast<const uint32_t*>(sp));
}

// Activations (a few hundred KB, shared by every workgroup: cached loads).
__device__ __forceinline__ Ops load_x(const uint8_t* p, const uint8_t* sp, bool valid) {
  if (!valid) {
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    return ops_from(z, z, z, z, z, z, 0x7f7f7f7fu);
  }
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  return ops_from(q[0], q[1], q[2], q[3], q[4], q[5], *reinterpret_cast<const uint32_t*>(sp));
}

template <int WF, int XF>
__device__ __forceinline__ v4f mfma_group(v4f acc, const Ops& w, const Ops& x) {
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.s0, x.s0, acc, WF, XF, 0, (int)w.sc, 0, (int)x.sc);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.s1, x.s1, acc, WF, XF, 1, (int)w.sc, 1, (int)x.sc);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.s2, x.s2, acc, WF, XF, 2, (int)w.sc, 2, (int)x.sc);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.s3, x.s3, acc, WF, XF, 3, (int)w.sc, 3, (int)x.sc);
  return acc;
}

// grid: (ceil(N / 128), splits).  Each wave: 32 features (2 fragments) x one K-chunk.
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

  // this lane's rows: token r16 of the activations, features nbase + 16 f + r16 of the weights
  const bool xvalid = r16 < g.M;
  const int64_t kbyte0 = (int64_t)split * kchunk * 3 / 4 + 96 * q;
  const int kblk0 = split * (kchunk / 32) + 4 * q;
  const uint8_t* xp = g.x_codes + (int64_t)(xvalid ? r16 : 0) * rowbytes + kbyte0;
  const uint8_t* xs = g.x_scales + (int64_t)(xvalid ? r16 : 0) * kblocks + kblk0;
  const int n0 = min(nbase + r16, g.N - 1), n1 = min(nbase + 16 + r16, g.N - 1);
  const uint8_t* wp0 = g.w_codes + (int64_t)n0 * rowbytes + kbyte0;
  const uint8_t* wp1 = g.w_codes + (int64_t)n1 * rowbytes + kbyte0;
  const uint8_t* ws0 = g.w_scales + (int64_t)n0 * kblocks + kblk0;
  const uint8_t* ws1 = g.w_scales + (int64_t)n1 * kblocks + kblk0;

  v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  if (ngroups > 0) {
    Ops x = load_x(xp, xs, xvalid);
    Ops w0 = load_w(wp0, ws0);
    Ops w1 = load_w(wp1, ws1);
    for (int grp = 0; grp < ngroups; ++grp) {
      Ops xn = x, w0n = w0, w1n = w1;
      if (grp + 1 < ngroups) {  // next group's loads in flight during this group's MFMAs
        const int64_t bo = (int64_t)(grp + 1) * kGroupBytes;
        const int so = (grp + 1) * 16;
        w0n = load_w(wp0 + bo, ws0 + so);
        w1n = load_w(wp1 + bo, ws1 + so);
        xn = load_x(xp + bo, xs + so, xvalid);
      }
      acc0 = mfma_group<WF, XF>(acc0, w0, x);
      acc1 = mfma_group<WF, XF>(acc1, w1, x);
      x = xn;
      w0 = w0n;
      w1 = w1n;
    }
  }

  // lane holds features nbase + 16 f + 4 q + (0..3) for token r16
  if (r16 < g.M) {
    float* part = g.partial + ((int64_t)split * 16 + r16) * g.N;
#pragma unroll
    for (int f = 0; f < kFragsPerWave; ++f) {
      const v4f a = f == 0 ? acc0 : acc1;
      const int n = nbase + 16 * f + 4 * q;
      if (n + 4 <= g.N && (g.N & 3) == 0) {
        *reinterpret_cast<v4f*>(part + n) = a;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < g.N) part[n + i] = a[i];
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
