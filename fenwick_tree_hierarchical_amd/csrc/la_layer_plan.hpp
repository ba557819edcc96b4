// Shape checks and workspace plan of the Log-Linear Mamba-2 layer (host and
// device, pure C++17).  The layer is the Mamba-2 block with its SSM replaced
// by the log-linear operator and one more group of projected columns for the
// per-level weights ("Log-Linear Attention", Spanish summary, technical
// section 2, "Variantes", item 1: Mamba-2's selective gate combined with the
// hierarchical mask).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "la_plan.hpp"

namespace la {

// Kernel geometry shared by the planner and the kernels.
constexpr int kGemmTile = 256;     // output tile of the projection GEMM (rows and columns)
constexpr int kGemmKBytes = 64;    // bytes of one row of a K-slice of the GEMM
constexpr int kPrologueTokens = 64;  // tokens per workgroup of the conv/gate kernel
constexpr int kPrologueRun = 16;     // tokens one thread rolls the conv window over
constexpr int kNormTokens = 16;      // tokens per workgroup of the gate/norm kernel
constexpr int kMaxConvTaps = 4;

struct LayerPlan {
  int B = 0, H = 0, P = 0, N = 0, G = 0, K = 0, C = 0, L = 0, d_model = 0, dtype = 0, es = 0;
  int64_t T = 0, M = 0;
  int d_inner = 0, conv_dim = 0, d_in_proj = 0, ld_zx = 0;
  int vec = 0;          // elements per 16-byte granule
  int norm_slots = 0;   // token rows the gate/norm kernel works on at once
  float eps = 0.f;
  // column offsets inside one row of the input projection
  int col_z = 0, col_x = 0, col_b = 0, col_c = 0, col_dt = 0, col_lam = 0;
  size_t off_zx = 0, off_q = 0, off_k = 0, off_v = 0, off_loga = 0, off_lam = 0, off_o = 0, off_opws = 0;
  size_t off_taps = 0;  // the conv taps and bias as fp32, [conv_dim][kMaxConvTaps + 1]
  size_t off_y = 0;     // the normalised gated output, over v (dead by then)
  size_t ws_bytes = 0;
  FwdPlan op;           // the operator's plan
  bool empty() const { return M == 0; }
};

inline int plan_layer(int B, int64_t T, int d_model, int H, int P, int N, int G, int K, int C, int L, float eps,
                      int dtype, LayerPlan* out) {
  if (!out) return kEINVAL;
  if (B < 0 || T < 0 || d_model <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || K <= 0 || L <= 0) return kEINVAL;
  if (dtype != kF32 && dtype != kBF16) return kEDTYPE;
  if (!(eps >= 0.f) || eps > 1.f) return kEINVAL;
  if (H % G != 0 || K > kMaxConvTaps) return kESHAPE;
  LayerPlan p;
  p.B = B; p.T = T; p.d_model = d_model; p.H = H; p.P = P; p.N = N; p.G = G; p.K = K; p.C = C; p.L = L;
  p.eps = eps; p.dtype = dtype;
  p.es = dtype == kBF16 ? 2 : 4;
  p.vec = 16 / p.es;
  const int kg = kGemmKBytes / p.es;   // the GEMM's K-slice
  if ((int64_t)H * P > 4096 || (int64_t)d_model > 65536) return kESHAPE;
  p.d_inner = H * P;
  if (d_model % kg != 0 || p.d_inner % kg != 0) return kESHAPE;
  // the gate/norm kernel holds one token row of d_inner in at most 256 lanes
  const int row_granules = p.d_inner / p.vec;
  if (row_granules > 256) return kESHAPE;
  // token rows at once: the largest power of two that fits, at most kNormTokens
  p.norm_slots = 1;
  while (2 * p.norm_slots * row_granules <= 256 && 2 * p.norm_slots <= kNormTokens) p.norm_slots *= 2;
  if (((p.d_inner / G) % p.vec) != 0) return kESHAPE;
  p.conv_dim = p.d_inner + 2 * G * N;
  const int64_t dip = 2 * (int64_t)p.d_inner + 2 * (int64_t)G * N + H + (int64_t)H * L;
  if (dip > 0x7fffffff / 2) return kESHAPE;
  p.d_in_proj = (int)dip;
  p.ld_zx = (int)align_up((size_t)p.d_in_proj, 8);
  p.col_z = 0;
  p.col_x = p.d_inner;
  p.col_b = 2 * p.d_inner;
  p.col_c = p.col_b + G * N;
  p.col_dt = p.col_c + G * N;
  p.col_lam = p.col_dt + H;
  p.M = (int64_t)B * T;
  if (p.M > (int64_t)0x7fffffff) return kESHAPE;
  int rc = plan_fwd(B, H, T, N, P, C, dtype, L, &p.op);
  if (rc != kOK) return rc;
  if (p.M == 0) {
    *out = p;
    return kOK;
  }
  const size_t M = (size_t)p.M, BHT = (size_t)B * H * (size_t)T, BGT = (size_t)B * G * (size_t)T;
  size_t off = 0;
  p.off_zx = off;   off = align_up(off + M * p.ld_zx * p.es, 256);
  // q = C and k = B once per group of heads: the operator reads group h / (H / G)
  p.off_q = off;    off = align_up(off + BGT * N * p.es, 256);
  p.off_k = off;    off = align_up(off + BGT * N * p.es, 256);
  p.off_v = off;    off = align_up(off + BHT * P * p.es, 256);
  p.off_loga = off; off = align_up(off + BHT * 4, 256);
  p.off_lam = off;  off = align_up(off + BHT * L * 4, 256);
  p.off_o = off;    off = align_up(off + BHT * P * p.es, 256);
  p.off_opws = off; off = align_up(off + p.op.ws_bytes, 256);
  p.off_taps = off; off = align_up(off + (size_t)p.conv_dim * (kMaxConvTaps + 1) * 4, 256);
  p.off_y = p.off_v;   // M * d_inner == B H T P
  p.ws_bytes = off;
  *out = p;
  return kOK;
}

}  // namespace la
