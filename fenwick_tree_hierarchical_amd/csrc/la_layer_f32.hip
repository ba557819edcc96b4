// float32 instantiations of the Log-Linear Mamba-2 layer kernels.
#include "la_internal.hpp"
#include "la_layer_impl.hpp"

namespace la {
int launch_layer_pre_f32(const LayerPlan& p, const void* u, const void* in_proj, const LayerArgs& a, hipStream_t s) {
  return launch_layer_pre<false>(p, u, in_proj, a, s);
}
int launch_layer_post_f32(const LayerPlan& p, const void* out_proj, void* out, const LayerArgs& a, hipStream_t s) {
  return launch_layer_post<false>(p, out_proj, out, a, s);
}
}  // namespace la
