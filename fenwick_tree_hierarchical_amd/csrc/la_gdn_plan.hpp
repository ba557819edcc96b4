// Host-side planning for the log-linear Gated DeltaNet forward: argument
// checks, the Fenwick node tree carve-up of the workspace and the LDS
// carve-up of its kernels.  Pure C++17 (builds into CPU test programs too).
//
// Workspace: one node per aligned block of 2^m full chunks (m = 0, 1, ...),
// level by level; node (m, bh, x) covers chunks [x 2^m, (x+1) 2^m) of head bh
// and holds
//   pt   [D][D] fp32  the block's state at its last token, (d_v, d_k) order
//                     (sum over its keys s of Phi(end, s) beta_s k_s v_s^T)
//   psit [D][D] fp32  the block's transition without gates, transposed
//                     (the product of (I - beta_r k_r k_r^T) over its tokens)
//   gn        fp32    the block's log2 gate total
#pragma once

#include "la_plan.hpp"

namespace la {

constexpr int kGdnMaxTree = 32;   // tree levels (n_full_chunks < 2^31)
constexpr int kGdnThreads = 256;  // 4 waves per workgroup in every kernel

// LDS regions are all C x (max(C, D) + 4) floats: a 16-byte row pad keeps
// the 16 rows an operand fragment reads in different banks.
LA_HD constexpr int gdn_ld(int C, int D) { return (C > D ? C : D) + 4; }
LA_HD constexpr int gdn_region_bytes(int C, int D) { return (C * gdn_ld(C, D) * 4 + 255) / 256 * 256; }

// gdn_chunk_prep: K, beta-and-gate scaled V, beta-scaled K, K K^T (then U),
// T^T and W, plus the gate scan and beta of the chunk.
struct GdnPrepLds {
  int k, vs, kb, g, tt, w, b2, beta, total;
};
LA_HD constexpr GdnPrepLds gdn_prep_lds(int C, int D) {
  GdnPrepLds o{};
  const int r = gdn_region_bytes(C, D);
  const int v = (C * 4 + 255) / 256 * 256;
  int off = 0;
  o.k = off;  off += r;
  o.vs = off; off += r;
  o.kb = off; off += r;
  o.g = off;  off += r;    // K K^T, then U = T diag(beta gate) V
  o.tt = off; off += r;
  o.w = off;  off += r;
  o.b2 = off; off += v;
  o.beta = off; off += v;
  o.total = off;
  return o;
}

// gdn_chunk_output: Q (then the carried queries), K, V, Q K^T (then the
// second carried-query buffer), K K^T (then A-hat, then the masked tile),
// T^T, the chunk's lambda rows, gate scan and beta.
struct GdnOutLds {
  int q, k, v, s, a, tt, lam, b2, beta, total;
};
LA_HD constexpr GdnOutLds gdn_out_lds(int C, int D, int L) {
  GdnOutLds o{};
  const int r = gdn_region_bytes(C, D);
  const int v = (C * 4 + 255) / 256 * 256;
  int off = 0;
  o.q = off;  off += r;
  o.k = off;  off += r;
  o.v = off;  off += r;
  o.s = off;  off += r;
  o.a = off;  off += r;
  o.tt = off; off += r;
  o.lam = off; off += (C * L * 4 + 255) / 256 * 256;
  o.b2 = off; off += v;
  o.beta = off; off += v;
  o.total = off;
  return o;
}

struct GdnPlan {
  int B = 0, H = 0, D = 0, C = 0, L = 0, dtype = 0, log2C = 0;
  int64_t T = 0, BH = 0, n_chunks = 0, n_full = 0;
  int n_tree = 0;                       // levels m with at least one node
  int64_t lev_off[kGdnMaxTree] = {};    // first node of level m
  int64_t n_nodes = 0;
  size_t off_pt = 0, off_psit = 0, off_gn = 0, ws_bytes = 0;
  int lds_prep = 0, lds_out = 0;
};

// Checks and the plan.  L < 0 skips the level-count check (workspace query).
inline int plan_gdn(int B, int H, int64_t T, int dk, int dv, int C, int dtype, int L, GdnPlan* p) {
  if (!p) return kEINVAL;
  if (B < 0 || H < 0 || T < 0) return kEINVAL;
  if (dtype != kF32 && dtype != kBF16) return kEDTYPE;
  if (dk != dv) return kESHAPE;
  if (!(dk == 16 || dk == 32 || dk == 64)) return kESHAPE;
  if (!(C == 16 || C == 32 || C == 64)) return kESHAPE;
  if (T > (int64_t)0x7fffffff) return kESHAPE;
  if ((int64_t)B * H > (int64_t)0x7fffffff) return kESHAPE;
  if (L >= 0) {
    if (L > kMaxLevels) return kESHAPE;
    if (T > 0 && L < levels_needed(T)) return kESHAPE;
  }
  GdnPlan P;
  P.B = B; P.H = H; P.T = T; P.D = dk; P.C = C; P.dtype = dtype;
  P.L = L < 0 ? kMaxLevels : L;
  P.log2C = ilog2(C);
  P.BH = (int64_t)B * H;
  P.n_chunks = (T + C - 1) / C;
  P.n_full = T / C;
  if (P.n_chunks * P.BH > (int64_t)0x7fffffff) return kESHAPE;
  P.lds_prep = gdn_prep_lds(C, dk).total;
  P.lds_out = gdn_out_lds(C, dk, P.L).total;
  if (P.lds_prep > kLdsLimit || gdn_out_lds(C, dk, kMaxLevels).total > kLdsLimit) return kESHAPE;
  int64_t n = 0;
  P.n_tree = 0;
  for (int m = 0; m < kGdnMaxTree && (P.n_full >> m) >= 1; ++m) {
    P.lev_off[m] = n;
    n += P.BH * (P.n_full >> m);
    P.n_tree = m + 1;
  }
  P.n_nodes = n;
  const size_t DD = (size_t)dk * dv;
  size_t off = 0;
  if (n > 0) {
    P.off_pt = off;   off = align_up(off + (size_t)n * DD * 4, 256);
    P.off_psit = off; off = align_up(off + (size_t)n * DD * 4, 256);
    P.off_gn = off;   off = align_up(off + (size_t)n * 4, 256);
  }
  P.ws_bytes = (P.BH == 0 || T == 0) ? 0 : off;
  *p = P;
  return kOK;
}

}  // namespace la
