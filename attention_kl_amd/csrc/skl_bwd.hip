// Launchers of the KL backward kernels (the kernel template and its dispatch are in skl_bwd_impl.hpp).
#include "skl_bwd_impl.hpp"

namespace skl {

hipError_t launch_bwd_dq(const BwdArgs& a, int dtype, int dt, int ds, bool causal, bool teacher, hipStream_t s) {
  return bwd_dispatch<false, true>(a, dtype, dt, ds, causal, teacher, s);
}

hipError_t launch_bwd_dk(const BwdArgs& a, int dtype, int dt, int ds, bool causal, bool teacher, hipStream_t s) {
  return bwd_dispatch<false, false>(a, dtype, dt, ds, causal, teacher, s);
}

}  // namespace skl
