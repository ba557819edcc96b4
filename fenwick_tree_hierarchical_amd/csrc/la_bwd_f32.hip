// float32 instantiations of the backward kernels.
#include "la_bwd_impl.hpp"
#include "la_internal.hpp"

namespace la {
int launch_bwd_f32(const BwdPlan& p, const FwdArgs& fa, const BwdArgs& a, hipStream_t s, bool saved) {
  return launch_bwd_dtype<false>(p, fa, a, s, saved);
}
}  // namespace la
