// Measurement aid (not part of the attention-KL method): the dense bf16 MFMA rate this GPU
// sustains and the shader clock it runs at meanwhile.  It gives the bench a measured
// denominator next to the published peak.  Declared in include/streamkl_probe.h.
#include "streamkl_probe.h"

#include <hip/hip_runtime.h>

#include "skl_device.hpp"

namespace skl {

// Every wave runs four independent chains of v_mfma_f32_32x32x16_bf16 (no memory traffic inside the
// loop), reading the shader-clock counter (s_memtime) and the constant-rate counter (s_memrealtime)
// before and after.  Each lane writes the sum of its accumulators, so no chain can be dropped.
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* __restrict__ sink, unsigned long long* __restrict__ clk,
                                                         int iters) {
  const int lane = threadIdx.x & 63;
  // small operands (2^-8 and near it): 16 products of about 2^-16 per element and step stay far
  // from overflow over any iteration count a caller would ask for
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.00390625f * (1.0f + 0.0078125f * ((lane + i) & 7)));
    b[i] = (__bf16)(0.00390625f * (1.0f + 0.0078125f * ((lane * 3 + i) & 7)));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[2 * (size_t)blockIdx.x] = t1 - t0;
    clk[2 * (size_t)blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace skl

extern "C" int streamkl_probe_mfma(int nblocks, int iters, float* sink, unsigned long long* clocks,
                                   double* wall_clock_khz, void* hip_stream) {
  if (nblocks <= 0 || iters <= 0 || sink == nullptr || clocks == nullptr || wall_clock_khz == nullptr) return 1;
  int dev = 0, rate = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 3;
  if (hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 3;
  *wall_clock_khz = (double)rate;
  hipLaunchKernelGGL(skl::mfma_probe_kernel, dim3((unsigned)nblocks), dim3(256), 0, (hipStream_t)hip_stream, sink,
                     clocks, iters);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
