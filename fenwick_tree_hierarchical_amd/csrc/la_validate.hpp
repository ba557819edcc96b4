// Host-side argument checks of the C ABI, after the shape plan: null
// pointers, alignment, workspace size and decode-state capacity.  Pure C++17
// with no HIP calls, so CPU test programs (tests/cpp) drive it directly,
// under the address and undefined-behaviour sanitizers.  Every check runs
// before anything is enqueued; the first failing one decides the code.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/logattn.h"
#include "la_bwd_plan.hpp"
#include "la_gdn_plan.hpp"
#include "la_layer_plan.hpp"
#include "la_plan.hpp"

namespace la {

// The decode state passed to loglinear_fwd_state, for the plan of its forward.
inline int check_fwd_state(const FwdPlan& p, const la_state* st) {
  int rc = check_state_shape(st->B, st->H, st->dk, st->dv, st->S);
  if (rc != kOK) return rc;
  if (st->B != p.B || st->H != p.H || st->dk != p.D || st->dv != p.D) return kESHAPE;
  if (bit_length(p.T) > st->S) return kECAPACITY;
  if (p.BH > 0) {
    if (!st->slots || !st->scale) return kEINVAL;
    if (!aligned(st->slots, 16) || !aligned(st->scale, 4)) return kEALIGN;
  }
  return kOK;
}

// The tensors and workspace of a non-empty forward.
inline int check_fwd_buffers(const FwdPlan& p, const void* q, const void* k, const void* v, const float* log_a,
                             const float* lambda, const void* out, const void* ws, size_t ws_bytes) {
  if (!q || !k || !v || !log_a || !lambda || !out) return kEINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return kEALIGN;
  if (!aligned(log_a, 4) || !aligned(lambda, 4)) return kEALIGN;
  if (p.ws_bytes > 0) {
    if (!ws || ws_bytes < p.ws_bytes) return kEWORKSPACE;
    if (!aligned(ws, 256)) return kEALIGN;
  }
  return kOK;
}

// The tensors and workspace of a non-empty backward.
inline int check_bwd_buffers(const BwdPlan& P, const void* q, const void* k, const void* v, const float* log_a,
                             const float* lambda, const void* dout, const void* gq, const void* gk, const void* gv,
                             const float* gla, const float* glam, const void* ws, size_t ws_bytes) {
  if (!q || !k || !v || !log_a || !lambda || !dout) return kEINVAL;
  if (!gq || !gk || !gv || !gla || !glam) return kEINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(gq, 16) ||
      !aligned(gk, 16) || !aligned(gv, 16))
    return kEALIGN;
  if (!aligned(log_a, 4) || !aligned(lambda, 4) || !aligned(gla, 4) || !aligned(glam, 4)) return kEALIGN;
  if (!ws || ws_bytes < P.ws_bytes) return kEWORKSPACE;
  if (!aligned(ws, 256)) return kEALIGN;
  return kOK;
}

// The workspace of the forward whose nodes a backward reuses (the forward's
// plan: the same shapes, dtype, chunk and levels).
inline int check_saved_fwd(const FwdPlan& p, const void* fwd_ws, size_t fwd_ws_bytes) {
  if (p.ws_bytes > 0) {
    if (!fwd_ws || fwd_ws_bytes < p.ws_bytes) return kEWORKSPACE;
    if (!aligned(fwd_ws, 256)) return kEALIGN;
  }
  return kOK;
}

// The tensors and workspace of a non-empty Gated DeltaNet forward.
inline int check_gdn_buffers(const GdnPlan& p, const void* q, const void* k, const void* v, const float* log_a,
                             const float* beta, const float* lambda, const void* out, const void* ws,
                             size_t ws_bytes) {
  if (!q || !k || !v || !log_a || !beta || !lambda || !out) return kEINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return kEALIGN;
  if (!aligned(log_a, 4) || !aligned(beta, 4) || !aligned(lambda, 4)) return kEALIGN;
  if (!ws || ws_bytes < p.ws_bytes) return kEWORKSPACE;
  if (!aligned(ws, 256)) return kEALIGN;
  return kOK;
}

// One decode step: the state, its capacity for the merge at position t, and
// the per-step tensors (unchecked when B * H == 0).  *kstar receives the
// number of levels the step merges.
inline int check_decode(const la_state* st, const void* q, const void* k, const void* v, const float* a,
                        const float* lambda, const void* out, int dtype, int* kstar) {
  if (!st) return kEINVAL;
  if (dtype != kF32 && dtype != kBF16) return kEDTYPE;
  int rc = check_state_shape(st->B, st->H, st->dk, st->dv, st->S);
  if (rc != kOK) return rc;
  if (st->t < 0) return kEINVAL;
  *kstar = trailing_ones(st->t);
  if (*kstar + 1 > st->S || bit_length(st->t) > st->S) return kECAPACITY;
  if ((int64_t)st->B * st->H > 0) {
    if (!st->slots || !st->scale || !q || !k || !v || !a || !lambda || !out) return kEINVAL;
    if (!aligned(st->slots, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
      return kEALIGN;
    if (!aligned(st->scale, 4) || !aligned(a, 4) || !aligned(lambda, 4)) return kEALIGN;
  }
  return kOK;
}

// The input, output, weights and workspace of a non-empty layer forward.
inline int check_layer_buffers(const LayerPlan& p, const void* u, const la_mamba2_weights* w, const void* out,
                               const void* ws, size_t ws_bytes) {
  if (!w) return kEINVAL;
  if (!u || !out || !w->in_proj || !w->conv_w || !w->conv_b || !w->dt_bias || !w->A_log || !w->D || !w->lam_bias ||
      !w->norm_w || !w->out_proj)
    return kEINVAL;
  if (!aligned(u, 16) || !aligned(out, 16) || !aligned(w->in_proj, 16) || !aligned(w->norm_w, 16) ||
      !aligned(w->out_proj, 16))
    return kEALIGN;
  if (!aligned(w->conv_w, p.es) || !aligned(w->conv_b, p.es)) return kEALIGN;
  if (!aligned(w->dt_bias, 4) || !aligned(w->A_log, 4) || !aligned(w->D, 4) || !aligned(w->lam_bias, 4))
    return kEALIGN;
  if (!ws || ws_bytes < p.ws_bytes) return kEWORKSPACE;
  if (!aligned(ws, 256)) return kEALIGN;
  return kOK;
}

}  // namespace la
