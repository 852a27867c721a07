// Device-resident scratch of the allocation-free backward entry point (streamkl_bwd_noalloc): the
// grouped-key workspace of the key-owner kernels, in a fixed-size array of every GPU the library
// runs on, so that callers which cannot allocate device memory need not pass one.
#include <hip/hip_runtime.h>

#include <mutex>

#include "skl_kernels.hpp"

namespace skl {

// One copy per GPU, at its own address, held until the process ends.  Host code never uses this
// name as an address (on the host it is only a stand-in for the symbol): scratch_address() resolves
// the device copy once per device and every launch receives that pointer.
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_address(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    // the current device is `dev`: this resolves that device's copy of the array
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace skl
