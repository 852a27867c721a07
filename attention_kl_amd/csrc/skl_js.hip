// Launchers of the Jensen-Shannon kernels: the forward's second pass and the two backward kernels
// (the kernel templates are in skl_fwd_impl.hpp and skl_bwd_impl.hpp, instantiated here with JS set).
#include "skl_bwd_impl.hpp"
#include "skl_fwd_impl.hpp"

namespace skl {

hipError_t launch_js_fwd(const FwdArgs& a, int dtype, int dt, int ds, bool causal, hipStream_t s) {
  return fwd_dispatch<true>(a, dtype, dt, ds, causal, s);
}

hipError_t launch_js_bwd_dq(const BwdArgs& a, int dtype, int dt, int ds, bool causal, bool teacher, hipStream_t s) {
  return bwd_dispatch<true, true>(a, dtype, dt, ds, causal, teacher, s);
}

hipError_t launch_js_bwd_dk(const BwdArgs& a, int dtype, int dt, int ds, bool causal, bool teacher, hipStream_t s) {
  return bwd_dispatch<true, false>(a, dtype, dt, ds, causal, teacher, s);
}

}  // namespace skl
