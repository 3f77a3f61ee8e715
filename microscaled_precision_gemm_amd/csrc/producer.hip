// Quantize-once producer for gfx950: RMSNorm + adaptive-norm modulation + MX
// quantization into the tiled GEMM operand layout, in one kernel.
//
// The Krea 3 / MI355X post (section "Fusion cut intermediate memory traffic")
// fuses the modulation and RMSNorm that produce the projection and MLP inputs
// and quantizes the activations once.  Per row r of x [rows, d]:
//
//   inv = 1 / sqrt(mean_k x[r,k]^2 + eps)
//   y[r,k] = x[r,k] * inv * gamma[k] * (1 + scale[c,k]) + shift[c,k],  c = r / rows_per_cond
//
// then y is MX-quantized along the row (the rule of mx_quantize), written as
// the tiled operand layout.  The MI300X counterpart is the page "Creating
// Custom Kernels for the AMD MI300", section "Fused RMS Norm Kernel" (128-bit
// coalesced loads, one block per row, a block-wide reduction); here:
//
//  * bf16 rows of up to 3072 elements (rmsnorm_quantize_rows_kernel): the rows
//    stay in registers between the passes, so x is read from HBM once (see
//    that kernel).  Wider rows and fp32 sources take the two-pass kernel:
//  * one workgroup (4 waves) per 32-row group.  Pass 1: each wave reduces the
//    sum of squares of 8 rows with 16-byte loads (consecutive lanes on
//    consecutive bytes, up to eight loads in flight) and a wave-wide shuffle
//    reduction, and parks 1/rms in LDS.  Pass 2: the waves take the group's
//    128-element stages in turn, exactly as the tiled quantizer does (the chunk
//    of 32 rows x 128 is staged through LDS so each lane owns two whole
//    blocks of one row, and the wave's next chunk is loaded while this one is
//    converted), apply the norm and the modulation in fp32 and convert with
//    v_cvt_scalef32_2xpk16 (round to nearest even, saturating).
//  * the second read of the group's rows comes from the caches: a group is
//    32 rows (192 KB for d = 3072) and was streamed just before.
//  * all rows of a group share one conditioning row (rows_per_cond is a
//    multiple of 32), so the stage's gain and modulation vectors are folded
//    into one (a, b) pair per feature in LDS.
#include "grid_limits.h"
#include "internal.h"
#include "mx_device.h"

namespace mxg {

namespace {

constexpr int kPWaves = 4;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPass1Loads = 8;  // 16-byte loads per lane in flight in pass 1 (a 3072-wide bf16 row: 6)

template <bool F32>
struct PLayout {
  static constexpr int kRowSrc = F32 ? 512 : 256;  // source bytes of one row of a 128-element stage
  static constexpr int kRow = kRowSrc + 16;        // padded LDS row
  static constexpr int kPieces = kRowSrc / 16;
  static constexpr int kCopies = 32 * kPieces / 64;
  static constexpr int kEsize = F32 ? 4 : 2;
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// 8 consecutive source elements (one 16-byte piece of bf16, or two of fp32) as fp32
template <bool F32>
__device__ __forceinline__ void piece_to_f32(const u32x4& w, float (&f)[4 * (F32 ? 1 : 2)]) {
  if constexpr (F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(w[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(w[e] << 16);
      f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
}

// Conversion of one staged chunk (32 rows x 128 elements in LDS, rows
// L::kRow bytes apart) and its store into the tiled layout: lane (h, j) takes
// blocks 2h, 2h+1 of row j, y = x * inv * va[k] + vb[k] over the stage's
// features k, then the MX rule.
template <int FMT, bool F32>
__device__ __forceinline__ void convert_store_chunk(const ProducerArgs& a, const uint8_t* in, const float* va,
                                                    const float* vb, float inv, int grp, int stage, int lane) {
  using L = PLayout<F32>;
  const int j = lane & 31, h = lane >> 5;
  const int row = grp * 32 + j;
  const int kblocks = a.d / 32;
  v6u q[2];
  uint32_t sbyte[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int qb = 2 * h + t;
    const uint8_t* p = in + j * L::kRow + qb * 32 * L::kEsize;
    float y[32];
#pragma unroll
    for (int i = 0; i < 32 / (16 / L::kEsize); ++i) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(p + 16 * i);
      float f[4 * (F32 ? 1 : 2)];
      piece_to_f32<F32>(w, f);
#pragma unroll
      for (int e = 0; e < 4 * (F32 ? 1 : 2); ++e) {
        const int kk = qb * 32 + i * (16 / L::kEsize) + e;  // element within the stage
        y[i * (16 / L::kEsize) + e] = __builtin_fmaf(f[e] * inv, va[kk], vb[kk]);
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; e += 2) amax = absmax2(amax, y[e], y[e + 1]);
    const BlockScale s = scale_from_f32_bits<FMT>(__float_as_uint(amax));
    v16f even, odd;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      even[i] = y[2 * i];
      odd[i] = y[2 * i + 1];
    }
    v6u r = cvt_f32x2x16<FMT>(even, odd, s.scale);
    uint32_t byte = s.byte;
    if (s.nonfinite) r = v6u{0, 0, 0, 0, 0, 0};
    if (row >= a.rows || stage * 4 + qb >= kblocks) {  // padding
      r = v6u{0, 0, 0, 0, 0, 0};
      byte = 127u;
    }
    q[t] = r;
    sbyte[t] = byte;
  }
  // the 48 code bytes of row j in the planes of half h of chunk (stage, grp)
  const int64_t chunk = (int64_t)stage * a.groups + grp;
  uint8_t* half = a.codes + chunk * kChunkCodes + h * kHalfBytes;
  *reinterpret_cast<u32x4*>(half + kPlaneA + j * 16) = u32x4{q[0][0], q[0][1], q[0][2], q[0][3]};
  *reinterpret_cast<u32x2*>(half + kPlaneL + j * 8) = u32x2{q[0][4], q[0][5]};
  *reinterpret_cast<u32x2*>(half + kPlaneH + j * 8) = u32x2{q[1][0], q[1][1]};
  *reinterpret_cast<u32x4*>(half + kPlaneB + j * 16) = u32x4{q[1][2], q[1][3], q[1][4], q[1][5]};
  *reinterpret_cast<uint16_t*>(a.scales + chunk * kChunkScales + j * 4 + 2 * h) =
      (uint16_t)(sbyte[0] | (sbyte[1] << 8));
}

template <int FMT, bool F32>
__global__ __launch_bounds__(kPThreads) void rmsnorm_quantize_kernel(const ProducerArgs a) {
  using L = PLayout<F32>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_chunk[kPWaves * 32 * L::kRow];
  __shared__ __attribute__((aligned(16))) float lds_ab[kPWaves][2][128];
  __shared__ float lds_inv[32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = blockIdx.x;
  const uint8_t* src = static_cast<const uint8_t*>(a.x);
  const int d = a.d, stages = (d + kTileStageK - 1) / kTileStageK;

  // ---- pass 1: 1 / rms of the group's rows, 8 rows per wave
  constexpr int kElemsPerLoad = 16 / L::kEsize;   // 8 bf16 or 4 fp32 per lane and load
  constexpr int kSpan = 64 * kElemsPerLoad;       // elements one wave load covers
  for (int i = 0; i < 8; ++i) {
    const int jr = wave * 8 + i;
    const int row = grp * 32 + jr;
    float ss = 0.0f;
    if (row < a.rows) {
      const uint8_t* xr = src + (int64_t)row * a.ld_bytes;
      for (int k0 = 0; k0 < d; k0 += kPass1Loads * kSpan) {
        u32x4 w[kPass1Loads];
#pragma unroll
        for (int u = 0; u < kPass1Loads; ++u) {
          const int e = k0 + u * kSpan + lane * kElemsPerLoad;
          // plain (cached) loads: pass 2 reads the same rows again
          w[u] = e < d ? *reinterpret_cast<const u32x4*>(xr + (int64_t)e * L::kEsize) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kPass1Loads; ++u) {
          float f[4 * (F32 ? 1 : 2)];
          piece_to_f32<F32>(w[u], f);
#pragma unroll
          for (int e = 0; e < 4 * (F32 ? 1 : 2); ++e) ss = __builtin_fmaf(f[e], f[e], ss);
        }
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) lds_inv[jr] = row < a.rows ? 1.0f / __builtin_sqrtf(ss / (float)d + a.eps) : 0.0f;
  }
  __syncthreads();

  // ---- pass 2: stages of the group, one wave at a time per stage
  uint8_t* in = lds_chunk + wave * 32 * L::kRow;
  float* va = lds_ab[wave][0];
  float* vb = lds_ab[wave][1];
  const int64_t cond = a.rows_per_cond > 0 ? (int64_t)grp * 32 / a.rows_per_cond : 0;
  const float* sh = a.shift ? a.shift + cond * d : nullptr;
  const float* sc = a.scale ? a.scale + cond * d : nullptr;
  const float inv = lds_inv[lane & 31];
  // the chunk of 32 rows x 128 elements of stage `stage`, 16 bytes per lane and load
  auto load = [&](int stage, u32x4 (&v)[L::kCopies]) {
#pragma unroll
    for (int i = 0; i < L::kCopies; ++i) {
      const int c = 64 * i + lane;
      const int jr = c / L::kPieces, piece = c % L::kPieces;
      const int r = grp * 32 + jr;
      const int e = stage * kTileStageK + piece * (16 / L::kEsize);
      v[i] = u32x4{0u, 0u, 0u, 0u};
      if (r < a.rows && e < d)
        v[i] = *reinterpret_cast<const u32x4*>(src + (int64_t)r * a.ld_bytes + (int64_t)e * L::kEsize);
    }
  };
  u32x4 v[L::kCopies];
  if (wave < stages) load(wave, v);
  for (int stage = wave; stage < stages; stage += kPWaves) {
#pragma unroll
    for (int i = 0; i < L::kCopies; ++i) {
      const int c = 64 * i + lane;
      const int jr = c / L::kPieces, piece = c % L::kPieces;
      *reinterpret_cast<u32x4*>(in + jr * L::kRow + piece * 16) = v[i];
    }
    // the wave's next stage is in flight while this one is converted
    if (stage + kPWaves < stages) load(stage + kPWaves, v);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int k = stage * kTileStageK + 2 * lane + t;
      float fa = 0.0f, fb = 0.0f;
      if (k < d) {
        fa = a.gamma ? a.gamma[k] : 1.0f;
        if (sc) fa *= 1.0f + sc[k];
        fb = sh ? sh[k] : 0.0f;
      }
      va[2 * lane + t] = fa;
      vb[2 * lane + t] = fb;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    convert_store_chunk<FMT, F32>(a, in, va, vb, inv, grp, stage, lane);
    // the next stage reuses this wave's LDS rows
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
}

// ---- bf16 rows of up to 3072 elements: the rows stay in registers between
// the passes, so x is read from HBM once.  A workgroup takes half of a
// 32-row group (16 rows; two workgroups fit a CU, so one's loads overlap the
// other's conversion): eight waves of two whole rows each (piece p = 64 i +
// lane of a row: elements 8p .. 8p+7, i = 0..5).  Pass 1 sums the squares
// from the registers.  Pass 2 takes the stages eight at a time: every wave
// writes its rows' pieces of the eight stages into eight LDS chunks (one
// 16-byte write per register and row: the 64 lanes of register i cover stages
// 4i .. 4i+3), and after a barrier wave w converts stage b + w, one block per
// lane (row lane % 16, block lane / 16).
constexpr int kRWaves = 8;
constexpr int kRMaxD = 3072;
constexpr int kRHalf = 16;                // rows per workgroup
constexpr int kRRows = kRHalf / kRWaves;  // rows per wave
constexpr int kRLoads = kRMaxD / 512;     // 16-byte pieces per lane and row
constexpr int kRStages = kRMaxD / kTileStageK;

template <int FMT>
__global__ __launch_bounds__(64 * kRWaves, 2) void rmsnorm_quantize_rows_kernel(const ProducerArgs a) {
  constexpr int kRow = 256 + 16;  // padded LDS row of a staged chunk
  __shared__ __attribute__((aligned(16))) uint8_t lds_chunk[kRWaves][kRHalf * kRow];
  __shared__ __attribute__((aligned(16))) float lds_ab[kRWaves][2][128];
  __shared__ float lds_inv[kRHalf];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = blockIdx.x >> 1, r0 = (blockIdx.x & 1) * kRHalf;  // group, first row in it
  const uint8_t* src = static_cast<const uint8_t*>(a.x);
  const int d = a.d, kblocks = d / 32, stages = (d + kTileStageK - 1) / kTileStageK;

  u32x4 v[kRRows][kRLoads];
#pragma unroll
  for (int rr = 0; rr < kRRows; ++rr) {
    const int row = grp * 32 + r0 + wave * kRRows + rr;
    const uint8_t* xr = src + (int64_t)(row < a.rows ? row : 0) * a.ld_bytes;
#pragma unroll
    for (int i = 0; i < kRLoads; ++i) {
      const int e = (64 * i + lane) * 8;
      v[rr][i] = row < a.rows && e < d ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + (int64_t)e * 2))
                                       : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // ---- pass 1
#pragma unroll
  for (int rr = 0; rr < kRRows; ++rr) {
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kRLoads; ++i) {
      float f[8];
      piece_to_f32<false>(v[rr][i], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
    }
    ss = wave_sum(ss);
    const int jr = wave * kRRows + rr, row = grp * 32 + r0 + jr;
    if (lane == 0) lds_inv[jr] = row < a.rows ? 1.0f / __builtin_sqrtf(ss / (float)d + a.eps) : 0.0f;
  }
  __syncthreads();

  // ---- pass 2
  const int j = lane & 15, q = lane >> 4;  // conversion: row j of the half-group, block q of the stage
  const int row = grp * 32 + r0 + j;
  const float inv = lds_inv[j];
  const int64_t cond = a.rows_per_cond > 0 ? (int64_t)grp * 32 / a.rows_per_cond : 0;
  const float* sh = a.shift ? a.shift + cond * d : nullptr;
  const float* sc = a.scale ? a.scale + cond * d : nullptr;
  const int sub = lane >> 4, piece = lane & 15;  // staging: stage 4i + sub of register i, its piece `piece`
#pragma unroll
  for (int b = 0; b < kRStages; b += kRWaves) {
    if (b >= stages) break;
#pragma unroll
    for (int i = b / 4; i < (b + kRWaves) / 4; ++i)
#pragma unroll
      for (int rr = 0; rr < kRRows; ++rr)
        *reinterpret_cast<u32x4*>(&lds_chunk[(4 * i + sub) % kRWaves][(wave * kRRows + rr) * kRow + piece * 16]) =
            v[rr][i];
    const int stage = b + wave;
    float* va = lds_ab[wave][0];
    float* vb = lds_ab[wave][1];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int k = stage * kTileStageK + 2 * lane + t;
      float fa = 0.0f, fb = 0.0f;
      if (stage < stages && k < d) {
        fa = a.gamma ? a.gamma[k] : 1.0f;
        if (sc) fa *= 1.0f + sc[k];
        fb = sh ? sh[k] : 0.0f;
      }
      va[2 * lane + t] = fa;
      vb[2 * lane + t] = fb;
    }
    __syncthreads();
    if (stage < stages) {
      const uint8_t* p = lds_chunk[wave] + j * kRow + q * 64;
      float y[32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p + 16 * i);
        float f[8];
        piece_to_f32<false>(w, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[8 * i + e] = __builtin_fmaf(f[e] * inv, va[q * 32 + 8 * i + e], vb[q * 32 + 8 * i + e]);
      }
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 32; e += 2) amax = absmax2(amax, y[e], y[e + 1]);
      const BlockScale s = scale_from_f32_bits<FMT>(__float_as_uint(amax));
      v16f even, odd;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        even[i] = y[2 * i];
        odd[i] = y[2 * i + 1];
      }
      v6u r = cvt_f32x2x16<FMT>(even, odd, s.scale);
      uint32_t byte = s.byte;
      if (s.nonfinite) r = v6u{0, 0, 0, 0, 0, 0};
      if (row >= a.rows || stage * 4 + q >= kblocks) {  // padding
        r = v6u{0, 0, 0, 0, 0, 0};
        byte = 127u;
      }
      // block q of row r0 + j: even blocks in planes A + L, odd ones in H + B, of half q / 2
      const int jj = r0 + j;
      const int64_t chunk = (int64_t)stage * a.groups + grp;
      uint8_t* half = a.codes + chunk * kChunkCodes + (q >> 1) * kHalfBytes;
      if ((q & 1) == 0) {
        *reinterpret_cast<u32x4*>(half + kPlaneA + jj * 16) = u32x4{r[0], r[1], r[2], r[3]};
        *reinterpret_cast<u32x2*>(half + kPlaneL + jj * 8) = u32x2{r[4], r[5]};
      } else {
        *reinterpret_cast<u32x2*>(half + kPlaneH + jj * 8) = u32x2{r[0], r[1]};
        *reinterpret_cast<u32x4*>(half + kPlaneB + jj * 16) = u32x4{r[2], r[3], r[4], r[5]};
      }
      a.scales[chunk * kChunkScales + jj * 4 + q] = (uint8_t)byte;
    }
    // every wave has converted its chunk: the next batch may overwrite them
    __syncthreads();
  }
}

// bf16 rows of up to kRMaxD features take the register-resident kernel (two
// workgroups per 32-row group), the rest the two-pass kernel (one per group)
bool rows_kernel(int64_t d, bool f32) { return !f32 && d <= kRMaxD; }

template <int FMT>
void launch_fmt(const ProducerArgs& a, bool f32, hipStream_t stream) {
  const dim3 grid((unsigned)a.groups), block(kPThreads);
  if (rows_kernel(a.d, f32))
    hipLaunchKernelGGL((rmsnorm_quantize_rows_kernel<FMT>), dim3(2 * (unsigned)a.groups), dim3(64 * kRWaves), 0,
                       stream, a);
  else if (f32)
    hipLaunchKernelGGL((rmsnorm_quantize_kernel<FMT, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((rmsnorm_quantize_kernel<FMT, false>), grid, block, 0, stream, a);
}

}  // namespace

int64_t rmsnorm_quantize_grid_items(int64_t rows, int64_t d, int src_type) {
  const int64_t groups = ceil_div(rows, kTileGroupRows);
  return rows_kernel(d, src_type == kSrcF32) ? 2 * groups * 64 * kRWaves : groups * kPThreads;
}

hipError_t launch_rmsnorm_quantize(const ProducerArgs& a, int src_type, int fmt, hipStream_t stream) {
  if (a.groups == 0 || a.d == 0) return hipSuccess;
  if (rmsnorm_quantize_grid_items(a.rows, a.d, src_type) > kMaxGridItems) return hipErrorInvalidConfiguration;
  if (fmt == kFmtE2M3)
    launch_fmt<kFmtE2M3>(a, src_type == kSrcF32, stream);
  else
    launch_fmt<kFmtE3M2>(a, src_type == kSrcF32, stream);
  return hipGetLastError();
}

}  // namespace mxg
