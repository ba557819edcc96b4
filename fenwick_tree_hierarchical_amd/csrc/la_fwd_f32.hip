// float32 instantiations of the forward kernels.
#include "la_fwd_impl.hpp"
#include "la_internal.hpp"

namespace la {
int launch_fwd_f32(const FwdPlan& p, const FwdArgs& a, hipStream_t s, hipEvent_t const* ev) {
  return launch_fwd_dtype<false>(p, a, s, ev);
}
}  // namespace la
