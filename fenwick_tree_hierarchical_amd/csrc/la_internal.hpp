// Internal launch entry points of liblogattn (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/logattn.h"
#include "la_bwd_plan.hpp"
#include "la_gdn_plan.hpp"
#include "la_layer_plan.hpp"
#include "la_plan.hpp"

namespace la {

struct FwdArgs;
struct BwdArgs;
struct GdnArgs;
struct LayerArgs;

// Forward: enqueue the stages of `p` on stream s; ev (nullable) holds
// p.n_stages + 1 events recorded around the stages.
int launch_fwd_bf16(const FwdPlan& p, const FwdArgs& a, hipStream_t s, hipEvent_t const* ev);
int launch_fwd_f32(const FwdPlan& p, const FwdArgs& a, hipStream_t s, hipEvent_t const* ev);

// Backward: enqueue its kernels on stream s.  fa carries the forward-structure
// buffers over (k := v, v := k).
int launch_bwd_bf16(const BwdPlan& p, const FwdArgs& fa, const BwdArgs& a, hipStream_t s, bool saved);
int launch_bwd_f32(const BwdPlan& p, const FwdArgs& fa, const BwdArgs& a, hipStream_t s, bool saved);

// Log-linear Gated DeltaNet forward: enqueue its kernels on stream s.
int launch_gdn_bf16(const GdnPlan& p, const GdnArgs& a, hipStream_t s);
int launch_gdn_f32(const GdnPlan& p, const GdnArgs& a, hipStream_t s);

// Log-Linear Mamba-2 layer: the input projection and the operator's inputs
// (pre), then the gate, norm and output projection (post).
int launch_layer_pre_bf16(const LayerPlan& p, const void* u, const void* in_proj, const LayerArgs& a, hipStream_t s);
int launch_layer_pre_f32(const LayerPlan& p, const void* u, const void* in_proj, const LayerArgs& a, hipStream_t s);
int launch_layer_post_bf16(const LayerPlan& p, const void* out_proj, void* out, const LayerArgs& a, hipStream_t s);
int launch_layer_post_f32(const LayerPlan& p, const void* out_proj, void* out, const LayerArgs& a, hipStream_t s);

int launch_decode(const la_state* st, const void* q, const void* k, const void* v, const float* a,
                  const float* lam, void* out, int dtype, int kstar, hipStream_t s);
int launch_state_init(float* slots, int64_t n_slots, float* scale, int64_t n_scale, hipStream_t s);
int launch_level_table(int64_t T, int log2C, int8_t* out, hipStream_t s);

}  // namespace la
