// Launcher of the KL forward kernel (the kernel template and its dispatch are in skl_fwd_impl.hpp).
#include "skl_fwd_impl.hpp"

namespace skl {

hipError_t launch_fwd(const FwdArgs& a, int dtype, int dt, int ds, bool causal, hipStream_t s) {
  return fwd_dispatch<false>(a, dtype, dt, ds, causal, s);
}

}  // namespace skl
