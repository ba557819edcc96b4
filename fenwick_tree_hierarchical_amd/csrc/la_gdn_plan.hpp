// Host-side planning for the log-linear Gated DeltaNet forward: argument
// checks, the Fenwick node tree carve-up of the workspace and the LDS
// carve-up of its kernels.  Pure C++17 (builds into CPU test programs too).
//
// Workspace, all per head bh:
//   tb   [n_chunks][C][C]  layer dtype  (T diag(beta))^T of every chunk, T
//                          the inverse of I + strict_tril(diag(beta) K K^T)
//   one node slot per aligned block of 2^m full chunks (m = 0, 1, ...), level
//   by level (odd level-0 slots are never written: no reader needs them);
//   node (m, bh, x) covers chunks [x 2^m, (x+1) 2^m) and holds
//   pt   [D][D]  layer dtype  the block's state at its last token, (d_v, d_k)
//                             order: sum over its keys s of
//                             Phi(end, s) beta_s k_s v_s^T, transposed
//   psit [D][D]  layer dtype  the block's transition without gates,
//                             transposed (the product of the
//                             I - beta_r k_r k_r^T over its tokens)
//   gn           fp32         the block's log2 gate total
#pragma once

#include "la_plan.hpp"

namespace la {

constexpr int kGdnMaxTree = 32;   // tree levels (n_full_chunks < 2^31)
constexpr int kGdnThreads = 512;     // 8 waves per workgroup: prep and tree kernels
constexpr int kGdnOutThreads = 256;  // 4 waves per workgroup: output kernel

// Row stride (elements) of an LDS tile with `cols` columns of es-byte
// elements: a 16-byte pad, so rows start 16-byte aligned and the rows one
// operand fragment reads spread over the banks.
LA_HD constexpr int gdn_lde(int cols, int es) { return cols + 16 / es; }
// Bytes of a rows x cols tile, rounded to 256.
LA_HD constexpr int gdn_tile(int rows, int cols, int es) { return (rows * gdn_lde(cols, es) * es + 255) / 256 * 256; }
LA_HD constexpr int gdn_max(int a, int b) { return a > b ? a : b; }

// gdn_chunk_prep: K row-major (then the solve's fp32 scratch, then U^T),
// K^T, (gated beta V)^T (then W^T) and (beta K)^T as swizzled token-major
// tiles, K K^T (fp32, then T in place), gate scan and beta; for the merge of
// a chunk pair, three D x D tiles from offset 0.
struct GdnPrepLds {
  int kr, kt, vst, kbt, g, b2, beta, total;
};
LA_HD constexpr GdnPrepLds gdn_prep_lds(int C, int D, int es) {
  GdnPrepLds o{};
  const int sw = (D * C * es + 255) / 256 * 256;                    // swizzled D x C tile
  const int f = gdn_tile(C, C, 4);                                  // fp32 C x C
  const int v = (C * 4 + 255) / 256 * 256;
  int off = 0;
  o.kr = off;  off += gdn_max(gdn_max(gdn_tile(C, D, es), gdn_tile(16, C, 4)), sw);
  o.kt = off;  off += sw;
  o.vst = off; off += sw;
  o.kbt = off; off += sw;
  o.g = off;   off += f;
  o.b2 = off;  off += v;
  o.beta = off; off += v;
  o.total = gdn_max(off, 3 * gdn_tile(D, D, es));
  return o;
}

// gdn_tree: Psi of the right half, row-major.
LA_HD constexpr int gdn_tree_lds(int D, int es) { return gdn_tile(D, D, es); }

// gdn_chunk_output (four waves): Q (then the carried queries), K (then
// Ahat), V (then the masked tile), tril(Q K^T) (then the second carried-query
// buffer), the chunk's lambda rows in the layer dtype, gate scan and beta.
// (T diag(beta))^T and the nodes are read from global memory into registers.
struct GdnOutLds {
  int q, k, v, s, lam, b2, beta, total;
};
LA_HD constexpr GdnOutLds gdn_out_lds(int C, int D, int es, int L) {
  GdnOutLds o{};
  const int cd = gdn_tile(C, D, es), cc = gdn_tile(C, C, es), mx = gdn_max(cd, cc);
  const int v = (C * 4 + 255) / 256 * 256;
  int off = 0;
  o.q = off;   off += cd;
  o.k = off;   off += mx;
  o.v = off;   off += mx;
  o.s = off;   off += mx;
  o.lam = off; off += (C * L * es + 255) / 256 * 256;
  o.b2 = off;  off += v;
  o.beta = off; off += v;
  o.total = off;
  return o;
}

struct GdnPlan {
  int B = 0, H = 0, D = 0, C = 0, L = 0, dtype = 0, es = 0, log2C = 0;
  int64_t T = 0, BH = 0, n_chunks = 0, n_full = 0;
  int n_tree = 0;                       // levels m with at least one node
  int64_t lev_off[kGdnMaxTree] = {};    // first node of level m
  int64_t n_nodes = 0;
  size_t off_tb = 0, off_pt = 0, off_psit = 0, off_gn = 0, ws_bytes = 0;
  int lds_prep = 0, lds_tree = 0, lds_out = 0;
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
  P.es = dtype == kBF16 ? 2 : 4;
  P.L = L < 0 ? kMaxLevels : L;
  P.log2C = ilog2(C);
  P.BH = (int64_t)B * H;
  P.n_chunks = (T + C - 1) / C;
  P.n_full = T / C;
  if (P.n_chunks * P.BH > (int64_t)0x7fffffff) return kESHAPE;
  P.lds_prep = gdn_prep_lds(C, dk, P.es).total;
  P.lds_tree = gdn_tree_lds(dk, P.es);
  P.lds_out = gdn_out_lds(C, dk, P.es, P.L).total;
  if (P.lds_prep > kLdsLimit || gdn_out_lds(C, dk, P.es, kMaxLevels).total > kLdsLimit) return kESHAPE;
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
  P.off_tb = off; off = align_up(off + (size_t)P.BH * P.n_chunks * C * C * P.es, 256);
  if (n > 0) {
    P.off_pt = off;   off = align_up(off + (size_t)n * DD * P.es, 256);
    P.off_psit = off; off = align_up(off + (size_t)n * DD * P.es, 256);
    P.off_gn = off;   off = align_up(off + (size_t)n * 4, 256);
  }
  P.ws_bytes = (P.BH == 0 || T == 0) ? 0 : off;
  *p = P;
  return kOK;
}

}  // namespace la
