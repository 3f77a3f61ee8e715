// Measurement only (libmxprobe.so, loaded by bench.py, not part of the GEMM
// library): the throughput the gfx950 scaled matrix instruction reaches with
// nothing else in the loop, on this board, with operands like the GEMM's.
//
// Each wave keeps eight 6-bit operand sets in registers (E2M3 codes of
// Gaussian-like data: random bits, which measured the same as quantized
// Gaussian blocks within 1 %), and issues V_MFMA_SCALE_F32_32X32X64_F8F6F4
// back to back on 16 accumulators, the way a 128 x 128 wave tile of the GEMM
// does (one operand kept for four instructions).  No memory traffic, no LDS,
// no epilogue: what it reaches is the matrix cores' rate under the board's
// power and clock limits for such data, the practical ceiling of any
// MFMA-bound kernel here.  Wave 0 of every workgroup also reads the shader
// clock counter (s_memtime) and the fixed 100 MHz counter (s_memrealtime) at
// the start and end of its loop, which gives the average engine clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <int FMT>
__global__ __launch_bounds__(256) void mfma_loop(int iters, uint32_t seed, float* sink, unsigned long long* clocks) {
  v8i a[4], b[4];
  uint32_t x = seed ^ ((blockIdx.x * 256u + threadIdx.x) * 2654435761u);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      x = x * 1664525u + 1013904223u;
      a[s][r] = (int)x;
      x = x * 1664525u + 1013904223u;
      b[s][r] = (int)x;
    }
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const unsigned long long t0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i / 4][i % 4] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i / 4], b[i % 4], acc[i / 4][i % 4], FMT,
                                                                         FMT, 0, 127, 0, 127);
  }
  const unsigned long long t1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[i][j][r];
  sink[blockIdx.x * 256 + threadIdx.x] = s;  // keeps the loop
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// Runs the loop on `workgroups` workgroups of 4 waves (one per SIMD; give the
// CU count for one wave per SIMD) for `iters` iterations of 16 instructions,
// `reps` times after one warm-up launch, on a stream of its own.  fmt: the
// instruction's format code (2 = E2M3, 4 = E2M1).  Writes the average time
// per launch (ms), the matrix-instruction rate (TFLOP/s) and the average
// engine clock of the last launch (GHz).  Returns 0, or -1 on a HIP error.
int mx_probe_mfma_ceiling(int fmt, int workgroups, int iters, int reps, double* ms, double* tflops, double* ghz) {
  if (workgroups <= 0 || iters <= 0 || reps <= 0 || !ms || !tflops || !ghz) return -1;
  if (fmt != 2 && fmt != 4) return -1;
  float* sink = nullptr;
  unsigned long long* clocks = nullptr;
  hipStream_t st = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = -1;
  if (hipMalloc(&sink, (size_t)workgroups * 256 * sizeof(float)) != hipSuccess) goto done;
  if (hipMalloc(&clocks, (size_t)workgroups * 2 * sizeof(unsigned long long)) != hipSuccess) goto done;
  if (hipStreamCreate(&st) != hipSuccess || hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess)
    goto done;
  for (int r = -1; r < reps; ++r) {
    if (r == 0 && hipEventRecord(e0, st) != hipSuccess) goto done;
    if (fmt == 2)
      hipLaunchKernelGGL(mfma_loop<2>, dim3(workgroups), dim3(256), 0, st, iters, 12345u + r, sink, clocks);
    else
      hipLaunchKernelGGL(mfma_loop<4>, dim3(workgroups), dim3(256), 0, st, iters, 12345u + r, sink, clocks);
    if (hipGetLastError() != hipSuccess) goto done;
  }
  if (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) goto done;
  {
    float t = 0.0f;
    if (hipEventElapsedTime(&t, e0, e1) != hipSuccess) goto done;
    unsigned long long c[2];
    if (hipMemcpy(c, clocks, sizeof(c), hipMemcpyDeviceToHost) != hipSuccess) goto done;
    *ms = (double)t / reps;
    *tflops = (double)workgroups * 4 * iters * 16 * 131072.0 / (*ms * 1e-3) / 1e12;
    *ghz = c[1] ? (double)c[0] / (double)c[1] * 0.1 : 0.0;
    rc = 0;
  }
done:
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (st) (void)hipStreamDestroy(st);
  if (sink) (void)hipFree(sink);
  if (clocks) (void)hipFree(clocks);
  return rc;
}

}  // extern "C"
