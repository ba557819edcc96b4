// Host-side plan of the backward pass: shape checks, the workspace carve-up
// and the LDS carve-up of the backward kernels.  Pure C++17 like la_plan.hpp,
// which it extends; the kernels include it so that LDS offsets are defined
// once.
#pragma once

#include "la_plan.hpp"

namespace la {

// bwd_chunk_dq and bwd_chunk_dkv: one workgroup per (b,h, chunk) of the
// forward output kernel's wave count.
LA_HD constexpr int bwd_waves(int C) { return output_waves(C); }

// LDS of the two per-chunk kernels.  Q, K, V and dout tiles are row-major with
// rows padded by 16 bytes; lam holds the chunk's lambda rows, b2 the
// in-chunk gate prefix.
//  bwd_chunk_dq: once the score tiles are formed, Q and V are dead: dS (by
//  query row) goes over V and the per-tile row sums of the lambda gradients
//  inside the chunk (part) over Q; after dq's intra-chunk product each wave's
//  share of the level gradients above the chunk (inter) goes over K and dS
//  when it fits.
//  bwd_chunk_dkv: dS^T and then P^T (by key row) in a region of their own
//  (s0), each wave's share of v . dv (col), and e2 the gate from each key to
//  the chunk end.
struct BwdChunkLds {
  int q, k, v, g, s0, lam, part, inter, col, b2, e2, total, ld_row, ld_s;
};
LA_HD constexpr BwdChunkLds bwd_chunk_lds(int C, int D, int es, int L, bool key_side) {
  BwdChunkLds o{};
  const int NW = bwd_waves(C);
  int log2c = 0;
  for (int c = C; c > 1; c >>= 1) ++log2c;
  o.ld_row = D + 16 / es;
  o.ld_s = C + 16 / es;
  const int tile = (C * o.ld_row * es + 255) / 256 * 256;
  const int stile = (C * o.ld_s * es + 255) / 256 * 256;
  const int vtile = key_side ? tile : (tile > stile ? tile : stile);
  int off = 0;
  o.q = off;  off += tile;
  o.k = off;  off += tile;
  o.v = off;  off += vtile;
  o.g = off;  off += tile;
  o.lam = off; off += (C * L * 4 + 255) / 256 * 256;
  o.b2 = off;  off += (C * 4 + 255) / 256 * 256;
  if (key_side) {
    o.s0 = off; off += stile;
    o.col = off; off += (NW * C * 4 + 255) / 256 * 256;
    o.e2 = off;  off += (C * 4 + 255) / 256 * 256;
    o.part = o.inter = -1;
  } else {
    o.s0 = o.v;
    o.part = o.q;          // fits: at most C/16 (C/16 + 1) / 2 * 64 + C/16 * 320 bytes
    o.inter = o.k;
    const int n_inter = L - log2c - 1 > 0 ? L - log2c - 1 : 0;
    const int inter_b = NW * n_inter * C * 4;
    if (inter_b > tile + vtile) { o.inter = off; off += (inter_b + 255) / 256 * 256; }
    o.col = o.e2 = -1;
  }
  o.total = off;
  return o;
}

// bwd_chunk_fused: both per-chunk kernels in one workgroup of twice the
// waves (the first half the query side, the second the key side), for the
// bf16 shapes where two such workgroups fit per CU.  Every buffer has a region
// of its own: the tiles, dS by query row (s0), dS^T and P^T by key row (s1,
// s2), lambda rows, the in-chunk and level shares of the lambda gradients
// (part, inter), the key side's shares of v . dv (col), the gate prefix (b2)
// and the gate from each key to the chunk end (e2).
struct BwdFusedLds {
  int q, k, v, g, s0, s1, s2, lam, part, inter, col, b2, e2, total, ld_row, ld_s;
};
LA_HD constexpr BwdFusedLds bwd_fused_lds(int C, int D, int es, int L) {
  BwdFusedLds o{};
  const int NW = bwd_waves(C);
  int log2c = 0;
  for (int c = C; c > 1; c >>= 1) ++log2c;
  o.ld_row = D + 16 / es;
  o.ld_s = C + 16 / es;
  const int tile = (C * o.ld_row * es + 255) / 256 * 256;
  const int stile = (C * o.ld_s * es + 255) / 256 * 256;
  const int QB = C / 16, NST = QB * (QB + 1) / 2;
  const int n_inter = L - log2c - 1 > 0 ? L - log2c - 1 : 0;
  int off = 0;
  o.q = off;  off += tile;
  o.k = off;  off += tile;
  o.v = off;  off += tile;
  o.g = off;  off += tile;
  o.s0 = off; off += stile;
  o.s1 = off; off += stile;
  o.s2 = off; off += stile;
  o.lam = off;   off += (C * L * 4 + 255) / 256 * 256;
  o.part = off;  off += ((NST * 16 + QB * 16 * 5) * 4 + 255) / 256 * 256;
  o.inter = off; off += (NW * n_inter * C * 4 + 255) / 256 * 256;
  o.col = off;   off += (NW * C * 4 + 255) / 256 * 256;
  o.b2 = off;    off += (C * 4 + 255) / 256 * 256;
  o.e2 = off;    off += (C * 4 + 255) / 256 * 256;
  o.total = off;
  return o;
}
// The fused kernel's shapes: bf16, 32 <= C (four waves per side), d <= 64.
LA_HD constexpr bool bwd_fused_shape(bool bf16, int C, int D) { return bf16 && C >= 32 && C <= 64 && D <= 64; }

// bwd_rev_states: one workgroup per (b,h, group of G chunks), the state
// kernel's wave count; gated Q^T and dout^T of one chunk, the group's gate
// prefixes and the chunk's token weights.
struct RevLds {
  int qt, gt, b2, w, total, ld_t;
};
LA_HD constexpr RevLds rev_lds(int C, int D, int es, int G) {
  RevLds o{};
  o.ld_t = C + 16 / es;
  const int tile = (D * o.ld_t * es + 255) / 256 * 256;
  int off = 0;
  o.qt = off; off += tile;
  o.gt = off; off += tile;
  o.b2 = off; off += (G * C * 4 + 255) / 256 * 256;
  o.w = off;  off += (C * 4 + 255) / 256 * 256;
  o.total = off;
  return o;
}

// bwd_rev_states_staged: one workgroup per half group (G / 2 chunks): the
// half's q and dout rows (bf16, swizzled row-major tiles), the gate prefixes
// of the whole group and two buffers of token weights.  Used where it fits
// twice per CU (d >= 64 for the swizzle, C >= 32 for the token k-step).
struct RevStagedLds {
  int q, g, b2, w, total;
};
LA_HD constexpr RevStagedLds rev_staged_lds(int C, int D, int G) {
  RevStagedLds o{};
  const int rows = (G / 2) * C * 2 * D;
  o.q = 0;
  o.g = rows;
  o.b2 = 2 * rows;
  o.w = o.b2 + G * C * 4;
  o.total = o.w + 2 * (G / 2) * C * 4;
  return o;
}
LA_HD constexpr bool rev_staged_fits(bool bf16, int C, int D, int G) {
  return bf16 && D >= 64 && C >= 32 && G >= 2 && 2 * rev_staged_lds(C, D, G).total <= kLdsLimit;
}
// The chunk-major walk of the same kernel (d = 64): the weight buffers become
// one table of the in-group levels and kRevGroupSlots group levels.
constexpr int kRevGroupSlots = 3;
LA_HD constexpr RevStagedLds rev_cm_lds(int C, int D, int G) {
  RevStagedLds o = rev_staged_lds(C, D, G);
  int log2g = 0;
  for (int g = G; g > 1; g >>= 1) ++log2g;
  o.total = o.w + (log2g + kRevGroupSlots) * (G / 2) * C * 4;
  return o;
}
LA_HD constexpr bool rev_cm_fits(bool bf16, int C, int D, int G) {
  return rev_staged_fits(bf16, C, D, G) && D == 64 && 2 * rev_cm_lds(C, D, G).total <= kLdsLimit;
}

struct BwdPlan {
  FwdPlan f;                 // the forward structure over (k := v, v := k): nodes for dq
  int JG = 0;                // group levels that have an upper block (bit length of n_groups - 1)
  int rhalves = 1;           // partial shares per group and level: 2 where the staged key-side kernel runs
  int lds_dq = 0, lds_dkv = 0, lds_rev = 0;
  int lds_fused = 0;         // > 0: the fused per-chunk kernel runs (two workgroups fit per CU)
  size_t off_rnodes_in = 0, off_rpart = 0, off_rnodes = 0, off_dcol = 0, ws_bytes = 0;
  // the same nodes transposed, (d_v, d_k), for the split key-side kernel
  // (the fused kernel gathers them from the columns of R); 0: not kept
  size_t off_rnodes_in_t = 0, off_rnodes_t = 0;
};

// Shape checks and the plan of the backward.  The forward's envelope, with
// chunks of at most 64 tokens; shapes whose tiles exceed the LDS are
// rejected.  L < 0 skips the level check (workspace query).
inline int plan_bwd(int B, int H, int64_t T, int dk, int dv, int C, int dtype, int L, BwdPlan* p) {
  if (!p) return kEINVAL;
  BwdPlan P;
  int rc = plan_fwd(B, H, T, dk, dv, C, dtype, L, &P.f);
  if (rc != kOK) return rc;
  if (C > 64) return kESHAPE;
  const FwdPlan& f = P.f;
  P.lds_dq = bwd_chunk_lds(C, dk, f.es, f.L, false).total;
  P.lds_dkv = bwd_chunk_lds(C, dk, f.es, f.L, true).total;
  P.lds_rev = rev_lds(C, dk, f.es, f.G).total;
  if (bwd_chunk_lds(C, dk, f.es, kMaxLevels, false).total > kLdsLimit ||
      bwd_chunk_lds(C, dk, f.es, kMaxLevels, true).total > kLdsLimit || P.lds_rev > kLdsLimit)
    return kESHAPE;
  if (bwd_fused_shape(f.es == 2, C, dk) && 2 * bwd_fused_lds(C, dk, f.es, f.L).total <= kLdsLimit)
    P.lds_fused = bwd_fused_lds(C, dk, f.es, f.L).total;
  if (f.BH == 0 || T == 0) {
    *p = P;
    return kOK;
  }
  P.JG = f.n_groups > 1 ? bit_length(f.n_groups - 1) : 0;
  P.rhalves = rev_staged_fits(f.es == 2, C, dk, f.G) ? 2 : 1;
  const size_t DD = (size_t)dk * dv;
  size_t off = f.ws_bytes;
  if (f.n_chunks > 1) {
    P.off_rnodes_in = off;   off = align_up(off + (size_t)f.BH * f.n_chunks * DD * f.es, 256);
    if (!P.lds_fused) {
      P.off_rnodes_in_t = off; off = align_up(off + (size_t)f.BH * f.n_chunks * DD * f.es, 256);
    }
  }
  if (f.n_groups > 1) {
    P.off_rpart = off;  off = align_up(off + (size_t)f.BH * f.n_groups * P.rhalves * P.JG * DD * 4, 256);
    P.off_rnodes = off;   off = align_up(off + (size_t)f.BH * f.n_groups * DD * f.es, 256);
    if (!P.lds_fused) {
      P.off_rnodes_t = off; off = align_up(off + (size_t)f.BH * f.n_groups * DD * f.es, 256);
    }
  }
  P.off_dcol = off; off = align_up(off + (size_t)f.BH * T * 4, 256);
  P.ws_bytes = off;
  *p = P;
  return kOK;
}

}  // namespace la
