// Measurement probe (not part of the attention library): the dense bf16 MFMA
// rate and the shader clock the chip sustains while it runs, for reporting
// kernel efficiency against both the published and the measured peak.
//
// Every wave issues `iters` rounds of 8 independent 32x32x16 bf16 MFMAs (8
// chains hide the instruction latency), so the SIMDs do nothing but matrix
// work.  Wave 0 of each workgroup brackets its loop with the shader clock
// counter (s_memtime) and the constant 100 MHz counter (s_memrealtime); their
// ratio gives the clock the SIMD ran at.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void mfma_clock_kernel(float* out, unsigned long long* clk,
                                                         int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (float)i);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = f32x16{};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[2 * (size_t)blockIdx.x] = t1 - t0;
    clk[2 * (size_t)blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// Flop of one launch: grid * 4 waves * iters * kChains MFMAs of 2*32*32*16.
double neoxprobe_mfma_flops(int grid, int iters) {
  return (double)grid * 4.0 * (double)iters * kChains * 2.0 * 32 * 32 * 16;
}

// Enqueues one probe launch on `stream`.  out: grid*256 floats; clk: 2*grid
// counters (shader-clock ticks, 100 MHz ticks) per workgroup.  Returns 0 on
// success, -1 for bad arguments, -5 when the launch fails.
int neoxprobe_mfma_launch(int grid, int iters, float* out, unsigned long long* clk,
                          void* stream) {
  if (grid < 1 || iters < 1 || !out || !clk) return -1;
  hipLaunchKernelGGL(mfma_clock_kernel, dim3((unsigned)grid), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), out, clk, iters);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
