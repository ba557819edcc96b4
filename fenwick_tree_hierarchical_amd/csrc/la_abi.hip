// C ABI of liblogattn: argument checks on the host, then launches.
// Every check happens before anything is enqueued; on error nothing runs.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/logattn.h"
#include "la_bwd_impl.hpp"
#include "la_fwd_impl.hpp"
#include "la_gdn_impl.hpp"
#include "la_internal.hpp"
#include "la_layer_impl.hpp"
#include "la_plan.hpp"
#include "la_validate.hpp"

using namespace la;

namespace {

// Kernel arguments of a non-empty forward over the workspace `w`.
FwdArgs fwd_args(const FwdPlan& p, const void* q, const void* k, const void* v, const float* log_a,
                 const float* lambda, void* out, char* w) {
  FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.log_a = log_a; a.lam = lambda; a.out = out;
  a.nodes_in = p.has_chunk_nodes() ? static_cast<void*>(w + p.off_nodes_in) : nullptr;
  a.gch = p.has_chunk_nodes() ? reinterpret_cast<float*>(w + p.off_gch) : nullptr;
  a.gstate = p.has_group_nodes() ? reinterpret_cast<float*>(w + p.off_gstate) : nullptr;
  a.gtot = p.has_group_nodes() ? reinterpret_cast<float*>(w + p.off_gtot) : nullptr;
  a.gprefix = p.has_group_nodes() ? reinterpret_cast<double*>(w + p.off_gprefix) : nullptr;
  a.nodes = p.has_group_nodes() ? static_cast<void*>(w + p.off_nodes) : nullptr;
  a.T = p.T; a.n_chunks = p.n_chunks; a.n_groups = p.n_groups; a.n_full_groups = p.n_full_groups; a.L = p.L;
  a.lam_vec4 = (p.T * p.L) % 4 == 0 && aligned(lambda, 16);
  return a;
}

// The forward; `st` (nullable) also receives the final recurrent state.
int fwd_common(const void* q, const void* k, const void* v, const float* log_a, const float* lambda,
               void* out, int B, int H, int64_t T, int dk, int dv, int C, int L, int dtype, void* ws,
               size_t ws_bytes, void* const* events, int n_events, la_state* st, la_stream_t stream) {
  FwdPlan p;
  int rc = plan_fwd(B, H, T, dk, dv, C, dtype, L, &p);
  if (rc != kOK) return rc;
  if (events && n_events != p.n_stages + 1) return kEINVAL;
  if (st) {
    rc = check_fwd_state(p, st);
    if (rc != kOK) return rc;
  }
  if (p.n_stages == 0) {   // empty problem: nothing to read or write
    if (events)
      for (int i = 0; i < n_events; ++i)
        if (hipEventRecord((hipEvent_t)events[i], (hipStream_t)stream) != hipSuccess) return kEHIP;
    if (st) {
      if (p.BH > 0) {      // T == 0: the state before any token
        rc = launch_state_init(st->slots, p.BH * st->S * dk * dv, st->scale, p.BH * st->S, (hipStream_t)stream);
        if (rc != kOK) return rc;
      }
      st->t = T;
    }
    return kOK;
  }
  rc = check_fwd_buffers(p, q, k, v, log_a, lambda, out, ws, ws_bytes);
  if (rc != kOK) return rc;
  FwdArgs a = fwd_args(p, q, k, v, log_a, lambda, out, static_cast<char*>(ws));
  a.st_slots = st ? st->slots : nullptr;
  a.st_scale = st ? st->scale : nullptr;
  a.st_S = st ? st->S : 0;
  const hipEvent_t* ev = reinterpret_cast<const hipEvent_t*>(events);
  hipStream_t s = (hipStream_t)stream;
  rc = dtype == kBF16 ? launch_fwd_bf16(p, a, s, ev) : launch_fwd_f32(p, a, s, ev);
  if (rc == kOK && st) st->t = T;
  return rc;
}

// The fixed scratch of loglinear_fwd_noalloc: a device array of the module,
// present on every GPU the library runs on.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol); it passes the device address hipGetSymbolAddress returns, looked
// up once per device, with that device current, on the first call there.
__device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the scratch array on the current device.
int scratch_on_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return kEHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return kEHIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return kOK;
}

}  // namespace

extern "C" {

LA_API const char* loglinear_strerror(int code) {
  switch (code) {
    case LA_OK: return "ok";
    case LA_EINVAL: return "invalid argument (null pointer or negative count)";
    case LA_ESHAPE: return "unsupported shape (head dim, chunk size, level count or size limit)";
    case LA_EDTYPE: return "unsupported dtype code";
    case LA_EALIGN: return "misaligned pointer";
    case LA_EWORKSPACE: return "workspace missing or too small";
    case LA_ECAPACITY: return "decode state has too few slots for this position";
    case LA_EHIP: return "HIP runtime or kernel launch error";
    case LA_ESCRATCH: return "problem needs more than the fixed scratch of loglinear_fwd_noalloc";
    default: return "unknown status code";
  }
}

LA_API int loglinear_version(void) { return 100; }

LA_API int loglinear_fwd_workspace(int B, int H, int64_t T, int dk, int dv, int C, int dtype,
                                   size_t* bytes) {
  if (!bytes) return kEINVAL;
  FwdPlan p;
  int rc = plan_fwd(B, H, T, dk, dv, C, dtype, -1, &p);
  if (rc != kOK) return rc;
  *bytes = p.ws_bytes;
  return kOK;
}

LA_API int loglinear_fwd_num_stages(int B, int H, int64_t T, int dk, int dv, int C, int dtype,
                                    int* n_stages) {
  if (!n_stages) return kEINVAL;
  FwdPlan p;
  int rc = plan_fwd(B, H, T, dk, dv, C, dtype, -1, &p);
  if (rc != kOK) return rc;
  *n_stages = p.n_stages;
  return kOK;
}

LA_API int loglinear_fwd(const void* q, const void* k, const void* v, const float* log_a,
                         const float* lambda, void* out, int B, int H, int64_t T, int dk, int dv,
                         int C, int L, int dtype, void* workspace, size_t workspace_bytes,
                         la_stream_t stream) {
  return fwd_common(q, k, v, log_a, lambda, out, B, H, T, dk, dv, C, L, dtype, workspace,
                    workspace_bytes, nullptr, 0, nullptr, stream);
}

LA_API int loglinear_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_a,
                                 const float* lambda, void* out, int B, int H, int64_t T, int dk,
                                 int dv, int C, int L, int dtype, la_stream_t stream) {
  FwdPlan p;
  int rc = plan_fwd(B, H, T, dk, dv, C, dtype, L, &p);
  if (rc != kOK) return rc;
  if (p.ws_bytes > LA_NOALLOC_SCRATCH_BYTES) return kESCRATCH;
  void* ws = nullptr;
  if (p.ws_bytes > 0) {
    rc = scratch_on_current_device(&ws);
    if (rc != kOK) return rc;
  }
  return fwd_common(q, k, v, log_a, lambda, out, B, H, T, dk, dv, C, L, dtype, ws, LA_NOALLOC_SCRATCH_BYTES,
                    nullptr, 0, nullptr, stream);
}

LA_API int loglinear_fwd_state(const void* q, const void* k, const void* v, const float* log_a,
                               const float* lambda, void* out, int B, int H, int64_t T, int dk, int dv,
                               int C, int L, int dtype, void* workspace, size_t workspace_bytes,
                               la_state* state, la_stream_t stream) {
  if (!state) return kEINVAL;
  return fwd_common(q, k, v, log_a, lambda, out, B, H, T, dk, dv, C, L, dtype, workspace,
                    workspace_bytes, nullptr, 0, state, stream);
}

LA_API int loglinear_fwd_staged(const void* q, const void* k, const void* v, const float* log_a,
                                const float* lambda, void* out, int B, int H, int64_t T, int dk,
                                int dv, int C, int L, int dtype, void* workspace,
                                size_t workspace_bytes, void* const* events, int n_events,
                                la_stream_t stream) {
  if (!events) return kEINVAL;
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return kEINVAL;
  return fwd_common(q, k, v, log_a, lambda, out, B, H, T, dk, dv, C, L, dtype, workspace,
                    workspace_bytes, events, n_events, nullptr, stream);
}

LA_API int loglinear_bwd_workspace(int B, int H, int64_t T, int dk, int dv, int C, int dtype,
                                   size_t* bytes) {
  if (!bytes) return kEINVAL;
  BwdPlan p;
  int rc = plan_bwd(B, H, T, dk, dv, C, dtype, -1, &p);
  if (rc != kOK) return rc;
  *bytes = p.ws_bytes;
  return kOK;
}

// The backward; with fwd_ws, the query side reads the nodes and gates of the
// caller's forward (its workspace) where the fused per-chunk kernel runs.
static int bwd_common(const void* q, const void* k, const void* v, const float* log_a, const float* lambda,
                      const void* dout, void* grad_q, void* grad_k, void* grad_v, float* grad_log_a,
                      float* grad_lambda, int B, int H, int64_t T, int dk, int dv, int C, int L, int dtype,
                      void* workspace, size_t workspace_bytes, const void* fwd_ws, size_t fwd_ws_bytes, bool from_fwd,
                      la_stream_t stream) {
  BwdPlan P;
  int rc = plan_bwd(B, H, T, dk, dv, C, dtype, L, &P);
  if (rc != kOK) return rc;
  const FwdPlan& p = P.f;
  if (p.BH == 0 || T == 0) return kOK;   // empty problem: nothing to read or write
  rc = check_bwd_buffers(P, q, k, v, log_a, lambda, dout, grad_q, grad_k, grad_v, grad_log_a, grad_lambda,
                         workspace, workspace_bytes);
  if (rc != kOK) return rc;
  if (from_fwd) {
    rc = check_saved_fwd(p, fwd_ws, fwd_ws_bytes);
    if (rc != kOK) return rc;
  }
  // the forward's nodes serve where the fused per-chunk kernel runs; elsewhere
  // the forward structure is built in this call's own workspace
  const bool saved = from_fwd && bwd_fused_shape(dtype == kBF16, C, dk) && P.lds_fused > 0;
  char* w = static_cast<char*>(workspace);
  char* n = saved ? static_cast<char*>(const_cast<void*>(fwd_ws)) : w;
  // forward structure over (k := v, v := k): its nodes are sum gate k v^T (the
  // forward's own nodes, over (k, v), are their transposes)
  FwdArgs fa{};
  fa.q = nullptr; fa.k = v; fa.v = k; fa.log_a = log_a; fa.lam = lambda; fa.out = nullptr;
  fa.nodes_in = p.has_chunk_nodes() ? static_cast<void*>(n + p.off_nodes_in) : nullptr;
  fa.gch = p.has_chunk_nodes() ? reinterpret_cast<float*>(n + p.off_gch) : nullptr;
  fa.gstate = p.has_group_nodes() ? reinterpret_cast<float*>(n + p.off_gstate) : nullptr;
  fa.gtot = p.has_group_nodes() ? reinterpret_cast<float*>(n + p.off_gtot) : nullptr;
  fa.gprefix = p.has_group_nodes() ? reinterpret_cast<double*>(n + p.off_gprefix) : nullptr;
  fa.nodes = p.has_group_nodes() ? static_cast<void*>(n + p.off_nodes) : nullptr;
  fa.T = T; fa.n_chunks = p.n_chunks; fa.n_groups = p.n_groups; fa.n_full_groups = p.n_full_groups; fa.L = L;
  BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.log_a = log_a; a.lam = lambda;
  a.dq = grad_q; a.dk = grad_k; a.dv = grad_v; a.dlog_a = grad_log_a; a.dlam = grad_lambda;
  a.nodes_in = fa.nodes_in; a.nodes = fa.nodes; a.gch = fa.gch; a.gprefix = fa.gprefix;
  a.rnodes_in = p.n_chunks > 1 ? static_cast<void*>(w + P.off_rnodes_in) : nullptr;
  a.rpart = p.n_groups > 1 ? reinterpret_cast<float*>(w + P.off_rpart) : nullptr;
  a.rnodes = p.n_groups > 1 ? static_cast<void*>(w + P.off_rnodes) : nullptr;
  a.rnodes_in_t = p.n_chunks > 1 && P.off_rnodes_in_t ? static_cast<void*>(w + P.off_rnodes_in_t) : nullptr;
  a.rnodes_t = p.n_groups > 1 && P.off_rnodes_t ? static_cast<void*>(w + P.off_rnodes_t) : nullptr;
  a.dcol = reinterpret_cast<float*>(w + P.off_dcol);
  a.T = T; a.n_chunks = p.n_chunks; a.n_groups = p.n_groups; a.L = L; a.JG = P.JG; a.rhalves = P.rhalves;
  hipStream_t s = (hipStream_t)stream;
  return dtype == kBF16 ? launch_bwd_bf16(P, fa, a, s, saved) : launch_bwd_f32(P, fa, a, s, saved);
}

LA_API int loglinear_bwd(const void* q, const void* k, const void* v, const float* log_a,
                         const float* lambda, const void* dout, void* grad_q, void* grad_k,
                         void* grad_v, float* grad_log_a, float* grad_lambda, int B, int H, int64_t T,
                         int dk, int dv, int C, int L, int dtype, void* workspace,
                         size_t workspace_bytes, la_stream_t stream) {
  return bwd_common(q, k, v, log_a, lambda, dout, grad_q, grad_k, grad_v, grad_log_a, grad_lambda, B, H, T, dk,
                    dv, C, L, dtype, workspace, workspace_bytes, nullptr, 0, false, stream);
}

LA_API int loglinear_bwd_from_fwd(const void* q, const void* k, const void* v, const float* log_a,
                                  const float* lambda, const void* dout, void* grad_q, void* grad_k,
                                  void* grad_v, float* grad_log_a, float* grad_lambda, int B, int H, int64_t T,
                                  int dk, int dv, int C, int L, int dtype, const void* fwd_workspace,
                                  size_t fwd_workspace_bytes, void* workspace, size_t workspace_bytes,
                                  la_stream_t stream) {
  return bwd_common(q, k, v, log_a, lambda, dout, grad_q, grad_k, grad_v, grad_log_a, grad_lambda, B, H, T, dk,
                    dv, C, L, dtype, workspace, workspace_bytes, fwd_workspace, fwd_workspace_bytes, true, stream);
}

LA_API int loglinear_gdn_fwd_workspace(int B, int H, int64_t T, int dk, int dv, int C, int dtype,
                                       size_t* bytes) {
  if (!bytes) return kEINVAL;
  GdnPlan p;
  int rc = plan_gdn(B, H, T, dk, dv, C, dtype, -1, &p);
  if (rc != kOK) return rc;
  *bytes = p.ws_bytes;
  return kOK;
}

LA_API int loglinear_gdn_fwd(const void* q, const void* k, const void* v, const float* log_a,
                             const float* beta, const float* lambda, void* out, int B, int H, int64_t T,
                             int dk, int dv, int C, int L, int dtype, void* workspace,
                             size_t workspace_bytes, la_stream_t stream) {
  GdnPlan p;
  int rc = plan_gdn(B, H, T, dk, dv, C, dtype, L, &p);
  if (rc != kOK) return rc;
  if (p.BH == 0 || T == 0) return kOK;   // empty problem: nothing to read or write
  rc = check_gdn_buffers(p, q, k, v, log_a, beta, lambda, out, workspace, workspace_bytes);
  if (rc != kOK) return rc;
  char* w = static_cast<char*>(workspace);
  GdnArgs a{};
  a.q = q; a.k = k; a.v = v; a.log_a = log_a; a.beta = beta; a.lam = lambda; a.out = out;
  a.tb = static_cast<void*>(w + p.off_tb);
  a.pt = p.n_nodes > 0 ? static_cast<void*>(w + p.off_pt) : nullptr;
  a.psit = p.n_nodes > 0 ? static_cast<void*>(w + p.off_psit) : nullptr;
  a.gn = p.n_nodes > 0 ? reinterpret_cast<float*>(w + p.off_gn) : nullptr;
  a.T = T; a.n_chunks = p.n_chunks; a.n_full = p.n_full; a.L = L;
  for (int m = 0; m < kGdnMaxTree; ++m) a.lev_off[m] = p.lev_off[m];
  hipStream_t s = (hipStream_t)stream;
  return dtype == kBF16 ? launch_gdn_bf16(p, a, s) : launch_gdn_f32(p, a, s);
}

LA_API int loglinear_state_bytes(int B, int H, int dk, int dv, int S, size_t* slot_bytes,
                                 size_t* scale_bytes) {
  if (!slot_bytes || !scale_bytes) return kEINVAL;
  int rc = check_state_shape(B, H, dk, dv, S);
  if (rc != kOK) return rc;
  *slot_bytes = (size_t)B * H * S * dk * dv * sizeof(float);
  *scale_bytes = (size_t)B * H * S * sizeof(float);
  return kOK;
}

LA_API int loglinear_state_init(la_state* st, int B, int H, int dk, int dv, int S, float* slots,
                                float* scale, la_stream_t stream) {
  if (!st) return kEINVAL;
  int rc = check_state_shape(B, H, dk, dv, S);
  if (rc != kOK) return rc;
  const int64_t BH = (int64_t)B * H;
  if (BH > 0) {
    if (!slots || !scale) return kEINVAL;
    if (!aligned(slots, 16) || !aligned(scale, 16)) return kEALIGN;
  }
  st->t = 0; st->B = B; st->H = H; st->dk = dk; st->dv = dv; st->S = S;
  st->slots = slots; st->scale = scale;
  if (BH == 0) return kOK;
  return launch_state_init(slots, BH * S * dk * dv, scale, BH * S, (hipStream_t)stream);
}

LA_API int loglinear_decode_step(la_state* st, const void* q, const void* k, const void* v,
                                 const float* a, const float* lambda, void* out, int dtype,
                                 la_stream_t stream) {
  int kstar = 0;
  int rc = check_decode(st, q, k, v, a, lambda, out, dtype, &kstar);
  if (rc != kOK) return rc;
  const int64_t BH = (int64_t)st->B * st->H;
  if (BH > 0) {
    rc = launch_decode(st, q, k, v, a, lambda, out, dtype, kstar, (hipStream_t)stream);
    if (rc != kOK) return rc;
  }
  st->t += 1;
  return kOK;
}

LA_API int loglinear_level_table(int64_t T, int C, int8_t* out, la_stream_t stream) {
  if (T < 1 || C < 1) return kEINVAL;
  if (T > kMaxTableT) return kESHAPE;
  if (!is_pow2(C) || C > (1 << 20)) return kESHAPE;
  if (!out) return kEINVAL;
  return launch_level_table(T, ilog2(C), out, (hipStream_t)stream);
}

}  // extern "C"

namespace {
int plan_layer_dims(const la_mamba2_dims* d, LayerPlan* p) {
  if (!d) return kEINVAL;
  return plan_layer(d->B, d->T, d->d_model, d->H, d->P, d->N, d->G, d->K, d->C, d->L, d->eps, d->dtype, p);
}
}  // namespace

extern "C" {

LA_API int loglinear_mamba2_fwd_workspace(const la_mamba2_dims* dims, size_t* bytes) {
  if (!bytes) return kEINVAL;
  LayerPlan p;
  const int rc = plan_layer_dims(dims, &p);
  if (rc != kOK) return rc;
  *bytes = p.ws_bytes;
  return kOK;
}

LA_API int loglinear_mamba2_fwd(const void* u, const la_mamba2_weights* weights, void* out,
                                const la_mamba2_dims* dims, void* workspace, size_t workspace_bytes,
                                la_stream_t stream) {
  LayerPlan p;
  int rc = plan_layer_dims(dims, &p);
  if (rc != kOK) return rc;
  if (p.empty()) return kOK;
  rc = check_layer_buffers(p, u, weights, out, workspace, workspace_bytes);
  if (rc != kOK) return rc;
  char* w = static_cast<char*>(workspace);
  LayerArgs a{};
  a.zx = w + p.off_zx;
  a.conv_w = weights->conv_w; a.conv_b = weights->conv_b;
  a.dt_bias = weights->dt_bias; a.A_log = weights->A_log; a.D = weights->D; a.lam_bias = weights->lam_bias;
  a.norm_w = weights->norm_w;
  a.taps = reinterpret_cast<float*>(w + p.off_taps);
  a.q = w + p.off_q; a.k = w + p.off_k; a.v = w + p.off_v;
  a.log_a = reinterpret_cast<float*>(w + p.off_loga);
  a.lam = reinterpret_cast<float*>(w + p.off_lam);
  a.o = w + p.off_o;
  a.y = w + p.off_y;
  a.T = p.T; a.H = p.H; a.P = p.P; a.N = p.N; a.G = p.G; a.K = p.K; a.L = p.L;
  a.d_inner = p.d_inner; a.conv_dim = p.conv_dim; a.ld_zx = p.ld_zx;
  a.col_x = p.col_x; a.col_b = p.col_b; a.col_c = p.col_c; a.col_dt = p.col_dt; a.col_lam = p.col_lam;
  a.norm_slots = p.norm_slots; a.eps = p.eps;
  FwdArgs fa = fwd_args(p.op, a.q, a.k, a.v, a.log_a, a.lam, w + p.off_o, w + p.off_opws);
  fa.qk_div = p.H / p.G;   // q and k are stored once per group of heads
  hipStream_t s = (hipStream_t)stream;
  const bool bf = p.dtype == kBF16;
  rc = bf ? launch_layer_pre_bf16(p, u, weights->in_proj, a, s) : launch_layer_pre_f32(p, u, weights->in_proj, a, s);
  if (rc != kOK) return rc;
  rc = bf ? launch_fwd_bf16(p.op, fa, s, nullptr) : launch_fwd_f32(p.op, fa, s, nullptr);
  if (rc != kOK) return rc;
  return bf ? launch_layer_post_bf16(p, weights->out_proj, out, a, s)
            : launch_layer_post_f32(p, weights->out_proj, out, a, s);
}

}  // extern "C"
