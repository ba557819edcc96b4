// f32 instantiations of the log-linear Gated DeltaNet forward kernels.
#include "la_gdn_impl.hpp"
#include "la_internal.hpp"

namespace la {
int launch_gdn_f32(const GdnPlan& p, const GdnArgs& a, hipStream_t s) { return launch_gdn_dtype<false>(p, a, s); }
}  // namespace la
