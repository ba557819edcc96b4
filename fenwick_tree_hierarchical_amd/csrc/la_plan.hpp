// Host-side planning for liblogattn: argument checks, the group size, the
// workspace carve-up and the LDS carve-up of each kernel.  Pure C++17 so that
// it builds both into the HIP library and into CPU-only test programs; the
// kernels include it too, so LDS offsets are defined in exactly one place.
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define LA_HD __host__ __device__
#else
#define LA_HD
#endif

namespace la {

enum : int { kF32 = 0, kBF16 = 1 };
enum : int {
  kOK = 0, kEINVAL = -1, kESHAPE = -2, kEDTYPE = -3, kEALIGN = -4,
  kEWORKSPACE = -5, kECAPACITY = -6, kEHIP = -7, kESCRATCH = -8
};

constexpr int kMaxLevels = 32;        // lambda levels accepted (T < 2^31 needs <= 32)
constexpr int kMaxDecodeSlots = 40;   // decode state slots (levels 1..S)
constexpr int kLdsLimit = 160 * 1024;  // gfx950 LDS per workgroup
constexpr int kWaves = 4;             // waves per workgroup in the forward kernels
constexpr int64_t kMaxTableT = 16384; // level-table export limit (T*T bytes)

LA_HD inline int ilog2(int64_t x) {   // floor(log2 x), x >= 1
  int r = 0;
  while (x > 1) { x >>= 1; ++r; }
  return r;
}
LA_HD inline int bit_length(int64_t x) {  // number of bits, 0 for x == 0
  int r = 0;
  while (x > 0) { x >>= 1; ++r; }
  return r;
}
inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Levels a sequence of length T uses: ceil(log2 T) + 1 (1 for T <= 1).
inline int levels_needed(int64_t T) { return T <= 1 ? 1 : bit_length(T - 1) + 1; }

// ---------------------------------------------------------------------------
// Kernel shapes shared by the host plan and the kernels.
//
// fwd_chunk_states: one workgroup per (b,h, group of G chunks); NW1 waves;
// each wave owns TPW of the (D/16)^2 tiles of a d_v x d_k state, and keeps
// the in-group Fenwick carry of those tiles in registers.
LA_HD constexpr int state_waves(int D) { return D <= 32 ? 4 : (D == 64 ? 8 : 16); }
LA_HD constexpr int state_tiles_per_wave(int D) {
  return ((D / 16) * (D / 16) + state_waves(D) - 1) / state_waves(D);
}
// Chunks per group: the largest power of two <= 8 whose carry (log2 G slots
// of TPW 16x16 fp32 tiles) fits in 32 registers per lane.
LA_HD constexpr int state_group(int D) {
  int G = 8;
  while (G > 1) {
    int ns = 0;
    for (int g = G; g > 1; g >>= 1) ++ns;
    if (ns * state_tiles_per_wave(D) * 4 <= 32) break;
    G >>= 1;
  }
  return G;
}
// fwd_chunk_output: one workgroup per (b,h, chunk) of max(C/16, 4) waves.
LA_HD constexpr int output_waves(int C) { return C / 16 > 4 ? C / 16 : 4; }

// LDS carve-up (byte offsets).  Tile rows are padded by 16 bytes so that the
// 16 rows one MFMA operand reads fall in different LDS banks.
// V^T and gated K^T of a chunk, double-buffered when both copies fit.
struct StateLds {
  int vt[2], kts[2], b2, total, ld_t, nbuf;
};
LA_HD constexpr StateLds state_lds(int C, int D, int es, int G) {
  StateLds o{};
  o.ld_t = C + 16 / es;
  const int tile = (D * o.ld_t * es + 255) / 256 * 256;
  const int b2 = (G * C * 4 + 255) / 256 * 256;
  o.nbuf = 4 * tile + b2 <= kLdsLimit / 2 ? 2 : 1;   // keep two workgroups per CU
  int off = 0;
  for (int b = 0; b < 2; ++b) {
    const int bb = b < o.nbuf ? b : 0;
    if (b < o.nbuf) {
      o.vt[b] = off;  off += tile;
      o.kts[b] = off; off += tile;
    } else {
      o.vt[b] = o.vt[bb];
      o.kts[b] = o.kts[bb];
    }
  }
  o.b2 = off;  off += b2;
  o.total = off;
  return o;
}
// bfloat16 tiles with 128- or 256-byte rows and C >= 32 arrive by direct global-to-LDS
// loads into unpadded rows whose 16-byte granules are XOR-permuted by the row
// index; the other shapes are staged through registers into padded rows.
LA_HD constexpr bool output_direct(int C, int D, int es) { return es == 2 && C >= 32 && (D == 64 || D == 128); }
struct OutLds {
  int q, k, v, p, lam, b2, e2, total, ld_row, ld_v, ld_p;
  bool direct;
};
LA_HD constexpr OutLds output_lds(int C, int D, int es, int L) {
  OutLds o{};
  o.direct = output_direct(C, D, es);
  o.ld_row = o.direct ? D : D + 16 / es;
  // staged V stays row-major; its rows are 4 bytes longer than a multiple of
  // 16, so the eight rows one V^T fragment gathers from fall in different banks
  o.ld_v = o.direct ? D : D + 4 / es;
  o.ld_p = C + 16 / es;
  int off = 0;
  o.q = off;    off += (C * o.ld_row * es + 255) / 256 * 256;
  // the masked score tile P is written over the K tile once K is dead
  o.k = off;
  o.p = off;
  {
    const int kb = C * o.ld_row * es, pb = C * o.ld_p * es;
    off += ((kb > pb ? kb : pb) + 255) / 256 * 256;
  }
  o.v = off;    off += (C * o.ld_v * es + 255) / 256 * 256;
  o.lam = off;  off += (C * L * 4 + 255) / 256 * 256;
  o.b2 = off;   off += (C * 4 + 255) / 256 * 256;
  o.e2 = off;   off += (C * 4 + 255) / 256 * 256;
  o.total = off;
  return o;
}
// The late-V variant of the output kernel (bfloat16, C = d = 64 or 128): the
// level contractions run before P V, so V is loaded into the Q tile once Q is
// dead and the workgroup needs one tile less (8 KB or 32 KB).
LA_HD constexpr bool output_vlate_shape(int C, int D, int es) { return es == 2 && ((C == 128 && D == 128) || (C == 64 && D == 64)); }
LA_HD constexpr OutLds output_lds_vlate(int C, int D, int es, int L) {
  OutLds o = output_lds(C, D, es, L);
  const int vbytes = (C * o.ld_v * es + 255) / 256 * 256;
  o.lam -= vbytes;
  o.b2 -= vbytes;
  o.e2 -= vbytes;
  o.total -= vbytes;
  o.v = o.q;
  return o;
}

struct FwdPlan {
  int B = 0, H = 0, D = 0, C = 0, L = 0, dtype = 0, es = 0;
  int64_t T = 0, BH = 0, n_chunks = 0, n_groups = 0;
  int64_t n_full_chunks = 0, n_full_groups = 0;   // chunks of C tokens, groups of G such chunks
  int G = 1, log2G = 0, log2C = 0;
  int lds_out = 0, lds_state = 0;
  int lds_out_vlate = 0;   // > 0: the late-V output kernel runs (two workgroups fit per CU)
  size_t off_nodes_in = 0, off_gch = 0;
  size_t off_gstate = 0, off_gtot = 0, off_gprefix = 0, off_nodes = 0, ws_bytes = 0;
  int n_stages = 0;   // 0 for an empty problem
  bool has_chunk_nodes() const { return n_full_chunks >= 1; }
  bool has_group_nodes() const { return n_full_groups >= 1; }
};

// Shape/dtype checks and the plan.  L < 0 skips the lambda-level check (used
// by the workspace query, which does not take L).
inline int plan_fwd(int B, int H, int64_t T, int dk, int dv, int C, int dtype, int L, FwdPlan* p) {
  if (!p) return kEINVAL;
  if (B < 0 || H < 0 || T < 0) return kEINVAL;
  if (dtype != kF32 && dtype != kBF16) return kEDTYPE;
  if (dk != dv) return kESHAPE;
  if (!(dk == 16 || dk == 32 || dk == 64 || dk == 128)) return kESHAPE;
  if (!(C == 16 || C == 32 || C == 64 || C == 128)) return kESHAPE;
  if (T > (int64_t)0x7fffffff) return kESHAPE;
  if ((int64_t)B * H > (int64_t)0x7fffffff) return kESHAPE;
  if (L >= 0) {
    if (L > kMaxLevels) return kESHAPE;
    if (T > 0 && L < levels_needed(T)) return kESHAPE;
  }
  FwdPlan P;
  P.B = B; P.H = H; P.T = T; P.D = dk; P.C = C; P.dtype = dtype;
  P.es = dtype == kBF16 ? 2 : 4;
  P.L = L < 0 ? kMaxLevels : L;
  P.BH = (int64_t)B * H;
  P.log2C = ilog2(C);
  P.G = state_group(dk);
  P.log2G = ilog2(P.G);
  P.lds_state = state_lds(C, dk, P.es, P.G).total;
  P.lds_out = output_lds(C, dk, P.es, P.L).total;
  if (output_vlate_shape(C, dk, P.es) && 2 * output_lds_vlate(C, dk, P.es, P.L).total <= kLdsLimit)
    P.lds_out_vlate = output_lds_vlate(C, dk, P.es, P.L).total;
  if (P.lds_state > kLdsLimit || output_lds(C, dk, P.es, kMaxLevels).total > kLdsLimit) return kESHAPE;
  P.n_chunks = (T + C - 1) / C;
  P.n_groups = (P.n_chunks + P.G - 1) / P.G;
  P.n_full_chunks = T / C;
  P.n_full_groups = P.n_full_chunks / P.G;
  if (P.n_chunks * P.BH > (int64_t)0x7fffffff) return kESHAPE;
  if (P.BH == 0 || T == 0) {
    P.n_stages = 0;
    *p = P;
    return kOK;
  }
  const size_t DD = (size_t)dk * dv;
  size_t off = 0;
  // chunk nodes exist once there is a full chunk, group nodes once there is a
  // full group (the forward reads them from the second chunk or group on; the
  // final state also reads those ending at the last full chunk and group)
  if (P.has_chunk_nodes()) {
    P.off_nodes_in = off; off = align_up(off + (size_t)P.BH * P.n_chunks * DD * P.es, 256);
    P.off_gch = off;      off = align_up(off + (size_t)P.BH * P.n_chunks * 4, 256);
  }
  if (P.has_group_nodes()) {
    P.off_gstate = off;  off = align_up(off + (size_t)P.BH * P.n_groups * DD * 4, 256);
    P.off_gtot = off;    off = align_up(off + (size_t)P.BH * P.n_groups * 4, 256);
    P.off_gprefix = off; off = align_up(off + (size_t)P.BH * (P.n_groups + 1) * 8, 256);
    P.off_nodes = off;   off = align_up(off + (size_t)P.BH * P.n_groups * DD * P.es, 256);
  }
  P.n_stages = P.n_groups > 1 ? 3 : (P.n_chunks > 1 ? 2 : 1);
  P.ws_bytes = off;
  *p = P;
  return kOK;
}

inline int check_state_shape(int B, int H, int dk, int dv, int S) {
  if (B < 0 || H < 0) return kEINVAL;
  if (dk != dv) return kESHAPE;
  if (!(dk == 16 || dk == 32 || dk == 64 || dk == 128)) return kESHAPE;
  if (S < 1 || S > kMaxDecodeSlots) return kESHAPE;
  if ((int64_t)B * H > (int64_t)0x7fffffff) return kESHAPE;
  return kOK;
}

// Trailing one bits of t: the number of levels a decode step at position t
// merges into level ctz(t+1)+1.
inline int trailing_ones(int64_t t) {
  int n = 0;
  while (t & 1) { t >>= 1; ++n; }
  return n;
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace la
