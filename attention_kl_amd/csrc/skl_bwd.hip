// Launchers of the KL backward kernels (the kernel template and its dispatch are in skl_bwd_impl.hpp).
#include "skl_bwd_impl.hpp"

namespace skl {

// Sum of the partial dK of a split group, in a fixed order (the result does not depend on timing).
__global__ __launch_bounds__(256) void sum_parts_kernel(float* __restrict__ dst, const float* __restrict__ parts,
                                                        int nsplit, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(parts + i);
    for (int k = 1; k < nsplit; ++k) acc += *reinterpret_cast<const f32x4*>(parts + k * n + i);
    *reinterpret_cast<f32x4*>(dst + i) = acc;
  }
}

// dK of each key head from the per-query-head contributions of its group, summed in head order:
// dst[r] = src[r G] + src[r G + 1] + ... (rows of `inner` floats; blockIdx.y = r).
__global__ __launch_bounds__(256) void group_sum_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                        int groups, int64_t inner) {
  const int64_t r = blockIdx.y;
  const float* s0 = src + r * groups * inner;
  float* d0 = dst + r * inner;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < inner; i += stride) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(s0 + i);
    for (int k = 1; k < groups; ++k) acc += *reinterpret_cast<const f32x4*>(s0 + k * inner + i);
    *reinterpret_cast<f32x4*>(d0 + i) = acc;
  }
}

hipError_t launch_group_sum(float* dst, const float* src, int64_t rows, int groups, int64_t inner, hipStream_t s) {
  if (rows <= 0 || inner <= 0) return hipSuccess;
  if (rows > 65535) return hipErrorInvalidValue;
  const int64_t want = (inner / 4 + 255) / 256;
  const unsigned gx = (unsigned)(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(group_sum_kernel, dim3(gx, (unsigned)rows), dim3(256), 0, s, dst, src, groups, inner);
  return hipGetLastError();
}

hipError_t launch_sum_parts(float* dst, const float* parts, int nsplit, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n / 4 + 255) / 256;
  const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(sum_parts_kernel, dim3(grid), dim3(256), 0, s, dst, parts, nsplit, n);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int dtype, int dt, int ds, bool causal, bool teacher, hipStream_t s) {
  return bwd_dispatch<false, true>(a, dtype, dt, ds, causal, teacher, s);
}

hipError_t launch_bwd_dk(const BwdArgs& a, int dtype, int dt, int ds, bool causal, bool teacher, hipStream_t s) {
  return bwd_dispatch<false, false>(a, dtype, dt, ds, causal, teacher, s);
}

}  // namespace skl
