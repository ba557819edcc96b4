// bfloat16 instantiations of the backward kernels.
#include "la_bwd_impl.hpp"
#include "la_internal.hpp"

namespace la {
int launch_bwd_bf16(const BwdPlan& p, const FwdArgs& fa, const BwdArgs& a, hipStream_t s, bool saved) {
  return launch_bwd_dtype<true>(p, fa, a, s, saved);
}
}  // namespace la
