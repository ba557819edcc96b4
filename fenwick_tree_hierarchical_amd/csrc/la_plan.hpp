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
  kEWORKSPACE = -5, kECAPACITY = -6, kEHIP = -7
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

// LDS carve-up of the forward kernels (byte offsets).  Rows of the bf16/f32
// tiles are padded by 16 bytes so that the 16 rows read by one MFMA operand
// fall in different LDS banks.
struct LdsLayout {
  int q, k, vt, kts, slots, lam, b2, ginfo, total;
  int ld_row;   // elements per row of the [C][D] tiles (Q, K)
  int ld_t;     // elements per row of the [D][C] tiles (VT, KTs)
  int ld_node;  // elements per row of a [D][D] node
};

constexpr int lds_take(int& off, int bytes) {
  const int r = off;
  off += (bytes + 255) / 256 * 256;
  return r;
}

// with_q: the output kernel (Q, K, lambda, chunk-level slots); otherwise the
// group-state kernel (V^T and the gated K^T only).
LA_HD constexpr LdsLayout lds_layout(int C, int D, int es, int G, int L, bool with_q) {
  LdsLayout o{};
  const int pad = 16 / es;
  o.ld_row = D + pad;
  o.ld_t = C + pad;
  o.ld_node = D + pad;
  int nslots = 0;                       // chunk levels 1..log2 G inside a group
  for (int g = G; g > 1; g >>= 1) ++nslots;
  int off = 0;
  o.q = with_q ? lds_take(off, C * o.ld_row * es) : -1;
  o.k = with_q ? lds_take(off, C * o.ld_row * es) : -1;
  o.vt = lds_take(off, D * o.ld_t * es);
  o.kts = (G > 1 || !with_q) ? lds_take(off, D * o.ld_t * es) : -1;
  o.slots = (with_q && nslots > 0) ? lds_take(off, nslots * D * o.ld_node * es) : -1;
  o.lam = with_q ? lds_take(off, C * L * 4) : -1;
  o.b2 = lds_take(off, G * C * 4);
  o.ginfo = with_q ? lds_take(off, 64 * 8) : -1;   // group-level node list
  o.total = off;
  return o;
}

// Chunks per workgroup of the output kernel: the largest power of two <= 8
// whose tiles fit in LDS with the largest accepted lambda stage; 0 if even a
// single chunk does not fit.
LA_HD constexpr int choose_group(int C, int D, int es) {
  for (int G = 8; G >= 1; G >>= 1)
    if (lds_layout(C, D, es, G, kMaxLevels, true).total <= (int)kLdsLimit) return G;
  return 0;
}

struct FwdPlan {
  int B = 0, H = 0, D = 0, C = 0, L = 0, dtype = 0, es = 0;
  int64_t T = 0, BH = 0, n_chunks = 0, n_groups = 0;
  int G = 1, log2G = 0, log2C = 0;
  int lds_out = 0, lds_state = 0;
  size_t off_gstate = 0, off_gtot = 0, off_gprefix = 0, off_nodes = 0, ws_bytes = 0;
  int n_stages = 0;   // 0 for an empty problem
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
  const int G = choose_group(C, dk, P.es);
  if (G == 0) return kESHAPE;
  P.G = G;
  P.log2G = ilog2(G);
  P.lds_out = lds_layout(C, dk, P.es, G, P.L, true).total;
  P.lds_state = lds_layout(C, dk, P.es, G, P.L, false).total;
  P.n_chunks = (T + C - 1) / C;
  P.n_groups = (P.n_chunks + G - 1) / G;
  if (P.BH == 0 || T == 0) {
    P.n_stages = 0;
    *p = P;
    return kOK;
  }
  const size_t DD = (size_t)dk * dv;
  size_t off = 0;
  if (P.n_groups > 1) {
    P.off_gstate = off; off = align_up(off + (size_t)P.BH * P.n_groups * DD * 4, 256);
    P.off_gtot = off;   off = align_up(off + (size_t)P.BH * P.n_groups * 4, 256);
    P.off_gprefix = off; off = align_up(off + (size_t)P.BH * (P.n_groups + 1) * 8, 256);
    P.off_nodes = off;  off = align_up(off + (size_t)P.BH * P.n_groups * DD * P.es, 256);
    P.n_stages = 3;
  } else {
    P.n_stages = 1;
  }
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
