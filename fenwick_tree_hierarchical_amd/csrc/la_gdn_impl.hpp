// Log-linear Gated DeltaNet forward on gfx950.
//
// Every Fenwick bucket state follows the gated delta rule's transition
// A_r = a_r (I - beta_r k_r k_r^T); the output is the lambda-weighted sum of
// the buckets ("Log-Linear Attention", both summaries, technical summary
// section 2: the framework laid over Gated DeltaNet).  Since the gates a_r
// are scalars, A_r = a_r Psi_r with Psi_r = I - beta_r k_r k_r^T, and inside
// one chunk of C tokens (gate log2-cumsum b, T = (I + strict_tril(diag(beta)
// K K^T))^-1) the compact product of the Psi_r gives:
//   * intra-chunk tile  Ahat = tril(Q K^T) T diag(beta):
//     Ahat[t,s] = beta_s q_t^T (Psi_t ... Psi_{s+1}) k_s, masked like the
//     Mamba-2 tile (lambda of the level, 2^(b_t - b_s)), then times V;
//   * carried queries   Q' = Q - Ahat K, so that a state P standing at the
//     chunk start is seen by query t as 2^(b_t) q'_t^T P;
//   * chunk node        P_c = K^T T diag(beta 2^(g - b)) V (state at chunk end)
//     and transition    Psi_c = I - K^T T diag(beta) K.
// Blocks of 2^m chunks merge as P = 2^(g_R) Psi_R P_L + P_R,
// Psi = Psi_R Psi_L.  For query chunk c the bucket nodes are the blocks of
// the set bits of c, most recent first; the queries are carried backwards
// through each block's Psi before meeting the next older node:
//   O_c += diag(lambda_lev 2^(b_t + G_j)) Q_j P_j,   Q_{j+1} = Q_j Psi_j,
// with G_j the log2 gates of the blocks between.
//
// Gates enter only as 2^x with x <= 0, taken by the hardware exponential
// (results below 2^-126 flush to zero).
//
// Kernels (8 waves per workgroup).  Tiles are staged in LDS in the layer
// dtype, with transposed copies where an operand is needed along its other
// axis, so that every matrix-core operand fragment is one contiguous load;
// the triangular solve and the accumulators are fp32.
//   gdn_chunk_prep    per pair of chunks: T by a blocked solve and
//                     (T diag(beta))^T for the output kernel; the nodes of
//                     full chunks (P_c, Psi_c, g_c), the even one stored, and
//                     their merge (the tree's level 1)
//   gdn_tree          per block of 2^m chunks, m >= 2: the merge of its halves
//   gdn_chunk_output  per chunk: the intra tile, the carried queries and the
//                     level contractions; writes the output.
#pragma once

#include "la_device.hpp"
#include "la_gdn_plan.hpp"

#include <type_traits>

namespace la {

struct GdnArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_a;
  const float* beta;
  const float* lam;
  void* out;
  void* tb;      // [BH][n_chunks][C][C] (T diag(beta))^T, layer dtype
  void* pt;      // [n_nodes][D][D] block states, (d_v, d_k) order, layer dtype
  void* psit;    // [n_nodes][D][D] block transitions without gates, transposed
  float* gn;     // [n_nodes] block log2 gate totals
  int64_t T;
  int64_t n_chunks;
  int64_t n_full;
  int L;
  int64_t lev_off[kGdnMaxTree];
};

constexpr int gdn_clog2(int x) { return x <= 1 ? 0 : 1 + gdn_clog2(x >> 1); }

// Operand fragments of the bf16 matrix cores: 8 consecutive k, from bf16 or
// fp32 storage.
struct GFrag {
  static __device__ __forceinline__ bf16x8 ld(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
  }
  static __device__ __forceinline__ bf16x8 ld(const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
    bf16x8 f;
    f[0] = (__bf16)a[0]; f[1] = (__bf16)a[1]; f[2] = (__bf16)a[2]; f[3] = (__bf16)a[3];
    f[4] = (__bf16)b[0]; f[5] = (__bf16)b[1]; f[6] = (__bf16)b[2]; f[7] = (__bf16)b[3];
    return f;
  }
  static __device__ __forceinline__ bf16x8 zero() {
    return __builtin_bit_cast(bf16x8, u16x8{0, 0, 0, 0, 0, 0, 0, 0});
  }
};

// acc += A[m0:m0+16, 0:K] B[0:K, n0:n0+16] on the matrix cores, with A stored
// A[m * lda + k] and B stored B[n * ldb + k] (both contiguous along k).
// Lane l supplies row/column l % 16 and the k-slice l / 16 of its operands;
// the result holds, in lane l, rows 4 (l / 16) + i of column l % 16, or with
// TR (operands swapped on the matrix cores) row l % 16 at the columns
// 4 (l / 16) + i.
template <bool BF16, int K, bool TR = false, typename TA, typename TB>
__device__ __forceinline__ f32x4 mm_kc(const TA* A, int lda, const TB* B, int ldb, int m0, int n0, f32x4 acc) {
  const int lane = lane_id(), r = lane & 15, kq = lane >> 4;
  if constexpr (BF16) {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
      const int kk = k0 + 8 * kq;
      bf16x8 fa = GFrag::zero(), fb = GFrag::zero();
      if (K >= 32 || kk < K) {
        fa = GFrag::ld(A + (m0 + r) * lda + kk);
        fb = GFrag::ld(B + (n0 + r) * ldb + kk);
      }
      acc = TR ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fa, acc, 0, 0, 0)
               : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4) {
      const float fa = A[(m0 + r) * lda + k0 + kq];
      const float fb = B[(n0 + r) * ldb + k0 + kq];
      acc = TR ? __builtin_amdgcn_mfma_f32_16x16x4f32(fb, fa, acc, 0, 0, 0)
               : __builtin_amdgcn_mfma_f32_16x16x4f32(fa, fb, acc, 0, 0, 0);
    }
  }
  return acc;
}

// The B-operand strip of one 16-column tile over all K, held in registers:
// the waves own fixed column strips of every product (n0 = 16 (wave % (N/16))
// for N <= 64), so a strip is loaded once and reused for all its row tiles,
// and one from global memory can be issued long before it is used.
template <bool BF16, int K> struct BStrip {
  static constexpr int N = BF16 ? (K + 31) / 32 : K / 4;
  typename std::conditional<BF16, bf16x8, float>::type f[N];
};
template <bool BF16, int K, typename TB>
__device__ __forceinline__ BStrip<BF16, K> load_strip(const TB* B, int ldb, int n0) {
  BStrip<BF16, K> b;
  const int lane = lane_id(), r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int s = 0; s < BStrip<BF16, K>::N; ++s) {
    if constexpr (BF16) {
      const int kk = 32 * s + 8 * kq;
      b.f[s] = (K >= 32 || kk < K) ? GFrag::ld(B + (n0 + r) * ldb + kk) : GFrag::zero();
    } else {
      b.f[s] = B[(n0 + r) * ldb + 4 * s + kq];
    }
  }
  return b;
}
template <bool BF16, int K, typename TA>
__device__ __forceinline__ f32x4 mm_strip(const TA* A, int lda, const BStrip<BF16, K>& b, int m0, f32x4 acc) {
  const int lane = lane_id(), r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int s = 0; s < BStrip<BF16, K>::N; ++s) {
    if constexpr (BF16) {
      const int kk = 32 * s + 8 * kq;
      const bf16x8 fa = (K >= 32 || kk < K) ? GFrag::ld(A + (m0 + r) * lda + kk) : GFrag::zero();
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, b.f[s], acc, 0, 0, 0);
    } else {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[(m0 + r) * lda + 4 * s + kq], b.f[s], acc, 0, 0, 0);
    }
  }
  return acc;
}

// The same product with the operands swapped (the strip as the A operand, the
// rows of A as the B operand): lane l then holds row m0 + l % 16 of the
// result at the four consecutive columns n0 + 4 (l / 16) + i, so a row weight
// is one value per lane and a row slice is one contiguous store.  Only the
// k-steps that overlap [klo, khi) are taken (wave-uniform bounds): the caller
// guarantees that both operands' other k contribute nothing (triangular
// factors).
template <bool BF16, int K, typename TA>
__device__ __forceinline__ f32x4 mm_strip_t(const TA* A, int lda, const BStrip<BF16, K>& b, int m0, f32x4 acc,
                                            int klo = 0, int khi = K) {
  const int lane = lane_id(), r = lane & 15, kq = lane >> 4;
  constexpr int KS = BF16 ? 32 : 4;
#pragma unroll
  for (int s = 0; s < BStrip<BF16, K>::N; ++s) {
    if (KS * s >= khi || KS * (s + 1) <= klo) continue;
    if constexpr (BF16) {
      const int kk = 32 * s + 8 * kq;
      const bf16x8 fa = (K >= 32 || kk < K) ? GFrag::ld(A + (m0 + r) * lda + kk) : GFrag::zero();
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.f[s], fa, acc, 0, 0, 0);
    } else {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(b.f[s], A[(m0 + r) * lda + 4 * s + kq], acc, 0, 0, 0);
    }
  }
  return acc;
}

// The B strip of a row-major tile M[s][n] taken along s (B[n][k] = M[k][n],
// n0 <= n < n0 + 16): scalar reads, once per wave, before M is reused.
template <bool BF16, int K, typename TB>
__device__ __forceinline__ BStrip<BF16, K> load_strip_t(const TB* M, int ldm, int n0) {
  BStrip<BF16, K> b;
  const int lane = lane_id(), r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int s = 0; s < BStrip<BF16, K>::N; ++s) {
    if constexpr (BF16) {
      const int kk = 32 * s + 8 * kq;
      bf16x8 f = GFrag::zero();
      if (K >= 32 || kk < K) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = __builtin_bit_cast(__bf16, M[(kk + i) * ldm + n0 + r]);
      }
      b.f[s] = f;
    } else {
      b.f[s] = M[(4 * s + kq) * ldm + n0 + r];
    }
  }
  return b;
}

// 16-byte vectors of a C x D row-major tile of global memory, rows at or
// past `nv` read as zero: every thread issues its loads before any is used.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <int C, int D, int ES, int NT = kGdnThreads> struct TileVec {
  static constexpr int EPV = 16 / ES, VPR = D / EPV, NV = C * VPR;
  static constexpr int VPT = (NV + NT - 1) / NT;
  u32x4 v[VPT];
};
// Thread-to-vector map: consecutive threads take consecutive rows of one
// 16-byte column, so that the transposed LDS copies written from the
// vectors land in consecutive addresses (no bank conflicts).
template <int C, int VPR>
__device__ __forceinline__ int tile_row(int e) { return e % C; }
template <int C, int VPR>
__device__ __forceinline__ int tile_vcol(int e) { return e / C; }
template <int C, int D, int NT = kGdnThreads, typename E>
__device__ __forceinline__ TileVec<C, D, sizeof(E), NT> load_tile(const E* p, int nv) {
  using TV = TileVec<C, D, sizeof(E), NT>;
  TV t;
#pragma unroll
  for (int u = 0; u < TV::VPT; ++u) {
    const int e = threadIdx.x + NT * u;
    const int i = tile_row<C, TV::VPR>(e), vc = tile_vcol<C, TV::VPR>(e);
    t.v[u] = u32x4{0u, 0u, 0u, 0u};
    if (e < TV::NV && i < nv) t.v[u] = reinterpret_cast<const u32x4*>(p)[i * TV::VPR + vc];
  }
  return t;
}
// The same with the coalesced map (eight consecutive threads read one
// 128-byte row whole), for tiles that are staged row-major.
template <int C, int VPR>
__device__ __forceinline__ int tile_row_c(int e) { return e / VPR; }
template <int C, int VPR>
__device__ __forceinline__ int tile_vcol_c(int e) { return e % VPR; }
template <int C, int D, int NT = kGdnThreads, typename E>
__device__ __forceinline__ TileVec<C, D, sizeof(E), NT> load_tile_c(const E* p, int nv) {
  using TV = TileVec<C, D, sizeof(E), NT>;
  TV t;
#pragma unroll
  for (int u = 0; u < TV::VPT; ++u) {
    const int e = threadIdx.x + NT * u;
    const int i = tile_row_c<C, TV::VPR>(e), vc = tile_vcol_c<C, TV::VPR>(e);
    t.v[u] = u32x4{0u, 0u, 0u, 0u};
    if (e < TV::NV && i < nv) t.v[u] = reinterpret_cast<const u32x4*>(p)[i * TV::VPR + vc];
  }
  return t;
}
// 16 bytes of E built from 16 / sizeof(E) floats.
template <typename E>
__device__ __forceinline__ u32x4 pack16(const float* x) {
  u32x4 w;
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (unsigned)Elem<true>::from_f32(x[2 * i]) | ((unsigned)Elem<true>::from_f32(x[2 * i + 1]) << 16);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_bit_cast(unsigned, x[i]);
  }
  return w;
}

// Element k of vector u of a loaded tile.
template <typename E, int C, int D, int NT = kGdnThreads>
__device__ __forceinline__ E tile_elem(const TileVec<C, D, sizeof(E), NT>& t, int u, int k) {
  if constexpr (sizeof(E) == 2) {
    const unsigned w = t.v[u][k >> 1];
    return static_cast<E>((k & 1) ? (w >> 16) : (w & 0xffffu));
  } else {
    const unsigned w = t.v[u][k];   // a scalar copy first: a bit cast of the
    return __builtin_bit_cast(E, w);  // vector element itself read element 0
  }
}

// Swizzled tile of rows of COLS elements with no padding: the 16-byte
// granule g of row m is stored at granule g ^ (m mod min(granules, 8)), so
// the rows an operand fragment reads at one granule fall in different banks.
template <typename E, int COLS>
__device__ __forceinline__ int swz(int m, int col) {
  constexpr int EPG = 16 / (int)sizeof(E), NG = COLS / EPG, GM = (NG < 8 ? NG : 8) - 1;
  return m * COLS + ((((col / EPG) ^ (m & GM)) * EPG) | (col % EPG));
}

// mm_kc with either operand in a swizzled [rows][K] tile (ASW / BSW); the
// other is stored contiguous along k with its leading dimension.
template <bool BF16, int K, bool ASW, bool BSW, bool TR = false, typename TA, typename TB>
__device__ __forceinline__ f32x4 mm_sw(const TA* A, int lda, const TB* B, int ldb, int m0, int n0, f32x4 acc) {
  const int lane = lane_id(), r = lane & 15, kq = lane >> 4;
  if constexpr (BF16) {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
      const int kk = k0 + 8 * kq;
      bf16x8 fa = GFrag::zero(), fb = GFrag::zero();
      if (K >= 32 || kk < K) {
        fa = GFrag::ld(A + (ASW ? swz<TA, K>(m0 + r, kk) : (m0 + r) * lda + kk));
        fb = GFrag::ld(B + (BSW ? swz<TB, K>(n0 + r, kk) : (n0 + r) * ldb + kk));
      }
      acc = TR ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fa, acc, 0, 0, 0)
               : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4) {
      const int k = k0 + kq;
      const float fa = A[ASW ? swz<TA, K>(m0 + r, k) : (m0 + r) * lda + k];
      const float fb = B[BSW ? swz<TB, K>(n0 + r, k) : (n0 + r) * ldb + k];
      acc = TR ? __builtin_amdgcn_mfma_f32_16x16x4f32(fb, fa, acc, 0, 0, 0)
               : __builtin_amdgcn_mfma_f32_16x16x4f32(fa, fb, acc, 0, 0, 0);
    }
  }
  return acc;
}

// The 16x16 output tiles of an M x N product dealt round-robin to the waves.
template <int M, int N, typename F>
__device__ __forceinline__ void for_tiles(F&& f) {
  constexpr int TN = N / 16, NT = (M / 16) * TN;
  for (int t = wave_id(); t < NT; t += kGdnThreads / 64) f((t / TN) * 16, (t % TN) * 16);
}

__device__ __forceinline__ int tile_row0() { return 4 * (lane_id() >> 4); }
__device__ __forceinline__ int tile_col() { return lane_id() & 15; }

template <typename E>
__device__ __forceinline__ E to_e(float x) { return Elem<sizeof(E) == 2>::from_f32(x); }
template <typename E>
__device__ __forceinline__ float from_e(E x) { return Elem<sizeof(E) == 2>::to_f32(x); }

// Four consecutive values of one output column, as one store / load.
template <typename E>
__device__ __forceinline__ void store4(E* p, f32x4 v) {
  if constexpr (sizeof(E) == 2) {
    *reinterpret_cast<u16x4*>(p) = u16x4{to_e<E>(v[0]), to_e<E>(v[1]), to_e<E>(v[2]), to_e<E>(v[3])};
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}
template <typename E>
__device__ __forceinline__ f32x4 load4(const E* p) {
  if constexpr (sizeof(E) == 2) {
    const u16x4 u = *reinterpret_cast<const u16x4*>(p);
    return f32x4{from_e<E>(u[0]), from_e<E>(u[1]), from_e<E>(u[2]), from_e<E>(u[3])};
  } else {
    return *reinterpret_cast<const f32x4*>(p);
  }
}

// T = (I + L)^-1 for the unit lower triangular I + L, L[i][m] = beta_i G[i][m]
// (m < i), row-major into Tm (fp32, zeros above the diagonal), by blocks of
// 16: the diagonal blocks by forward substitution (lane 16 b + j solves
// column j of block b), then each block row r from the rows above it,
// T_rj = -T_rr sum_{k<r} L_rk T_kj, on the fp32 matrix cores.  Called by every thread of the
// workgroup; returns with the workgroup synchronised.
template <int C>
__device__ __forceinline__ void solve_blocked(const float* G, const float* beta, float* Tm, float* X) {
  constexpr int LF = gdn_lde(C, 4), NB = C / 16;
  const int tid = threadIdx.x;
  for (int e = tid; e < C * C; e += kGdnThreads) {   // the blocks above the diagonal
    const int i = e / C, j = e % C;
    if ((j >> 4) > (i >> 4)) Tm[i * LF + j] = 0.f;
  }
  if (tid < 16 * NB) {
    const int b = tid >> 4, j = tid & 15, o = 16 * b;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p0 = 0.f, p1 = 0.f;   // two chains hide the FMA latency
#pragma unroll
      for (int m = 0; m + 1 < i; m += 2) {
        p0 = fmaf(G[(o + i) * LF + o + m], x[m], p0);
        p1 = fmaf(G[(o + i) * LF + o + m + 1], x[m + 1], p1);
      }
      if (i & 1) p0 = fmaf(G[(o + i) * LF + o + i - 1], x[i - 1], p0);
      x[i] = (i == j ? 1.f : 0.f) - beta[o + i] * (p0 + p1);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Tm[(o + i) * LF + o + j] = x[i];
  }
  __syncthreads();
  // block rows on the fp32 matrix cores (lane l supplies A[l % 16][l / 16]
  // and B[l / 16][l % 16] of each 16 x 16 x 4 step, passed swapped so that
  // lane l receives row l % 16 at the columns 4 (l / 16) + i): wave cb forms
  // X = beta L[rb, cb..rb-1] T[cb..rb-1, cb], then T[rb, cb] = -T[rb, rb] X
  const int w = wave_id(), lane = lane_id(), r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int rb = 1; rb < NB; ++rb) {
    const int o = 16 * rb;
    if (w < rb) {
      const int oc = 16 * w;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float br = beta[o + r];
      for (int kb = w; kb < rb; ++kb) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int k = 16 * kb + 4 * st + kq;
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Tm[k * LF + oc + r], G[(o + r) * LF + k] * br, acc, 0, 0, 0);
        }
      }
      *reinterpret_cast<f32x4*>(X + r * LF + oc + 4 * kq) = acc;
    }
    __syncthreads();
    if (w < rb) {
      const int oc = 16 * w;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int k = 4 * st + kq;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[k * LF + oc + r], Tm[(o + r) * LF + o + k], acc, 0, 0, 0);
      }
      *reinterpret_cast<f32x4*>(Tm + (o + r) * LF + oc + 4 * kq) = f32x4{-acc[0], -acc[1], -acc[2], -acc[3]};
    }
    __syncthreads();
  }
}

// Inclusive log2 gate prefix of the chunk starting at t0 and its betas, zero
// past `nv` valid tokens.  One wave.
template <int C>
__device__ __forceinline__ void gdn_gate_scan(const float* la, const float* be, int64_t t0, int nv, float* b2,
                                              float* bet) {
  const int l = lane_id();
  float x = (l < nv) ? la[t0 + l] * kLog2e : 0.f;
  x = wave_incl_scan(x);
  if (l < C) {
    b2[l] = x;
    bet[l] = (l < nv) ? be[t0 + l] : 0.f;
  }
}

// ---------------------------------------------------------------------------
// gdn_chunk_prep, one chunk: T by the blocked solve, (T diag(beta))^T written
// for the output kernel, and for a full chunk its node in registers: each
// wave holds NPW 16x16 tiles of the state (P) and of the transition (S),
// tile u being (m0, n0) = (16 (t / TN), 16 (t % TN)), t = wave + NW u, rows
// m0 + 4 (lane / 16) + i of column n0 + lane % 16.  Returns whether the chunk
// is full; `gout` is its log2 gate total.
template <int D> struct PrepTiles {
  static constexpr int TN = D / 16, NT = TN * TN, NW = kGdnThreads / 64, NPW = (NT + NW - 1) / NW;
};

template <bool BF16, int C, int D>
__device__ __forceinline__ bool gdn_prep_chunk(const GdnArgs& a, unsigned char* smem, int64_t bh, int64_t c,
                                               f32x4 (&P)[PrepTiles<D>::NPW], f32x4 (&S)[PrepTiles<D>::NPW],
                                               float& gout) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  constexpr int es = sizeof(E);
  constexpr int LDD = gdn_lde(D, es), LF = gdn_lde(C, 4);
  constexpr GdnPrepLds LY = gdn_prep_lds(C, D, es);
  // K row-major (padded), then the solve's scratch, then U^T; the token-major
  // tiles K^T, (gated beta V)^T (then W^T) and (beta K)^T are swizzled
  E* Kr = reinterpret_cast<E*>(smem + LY.kr);
  float* X = reinterpret_cast<float*>(smem + LY.kr);
  E* Ut = reinterpret_cast<E*>(smem + LY.kr);
  E* Kt = reinterpret_cast<E*>(smem + LY.kt);
  E* Vst = reinterpret_cast<E*>(smem + LY.vst);
  E* Wt = reinterpret_cast<E*>(smem + LY.vst);
  E* Kbt = reinterpret_cast<E*>(smem + LY.kbt);
  float* G = reinterpret_cast<float*>(smem + LY.g);   // K K^T, then T in place
  float* Tm = G;
  float* b2 = reinterpret_cast<float*>(smem + LY.b2);
  float* bet = reinterpret_cast<float*>(smem + LY.beta);
  const int64_t t0 = c * C;
  const int nv = (int)((a.T - t0) < C ? (a.T - t0) : C);
  const bool full = c < a.n_full;
  const int tid = threadIdx.x;
  using TV = TileVec<C, D, es>;
  const TV kt = load_tile<C, D>(static_cast<const E*>(a.k) + (bh * a.T + t0) * D, nv);
  const TV vt = load_tile<C, D>(static_cast<const E*>(a.v) + (bh * a.T + t0) * D, nv);
  if (wave_id() == 0) gdn_gate_scan<C>(a.log_a + bh * a.T, a.beta + bh * a.T, t0, nv, b2, bet);
  __syncthreads();
  const float g = b2[C - 1];
#pragma unroll
  for (int u = 0; u < TV::VPT; ++u) {
    const int e = tid + kGdnThreads * u;
    if (e < TV::NV) {
      const int i = tile_row<C, TV::VPR>(e), j0 = tile_vcol<C, TV::VPR>(e) * TV::EPV;
      *reinterpret_cast<u32x4*>(Kr + i * LDD + j0) = kt.v[u];
      const float sb = bet[i], sv = bet[i] * __builtin_amdgcn_exp2f(g - b2[i]);
#pragma unroll
      for (int kk = 0; kk < TV::EPV; ++kk) {
        const E ke = tile_elem<E, C, D>(kt, u, kk);
        const int at = swz<E, C>(j0 + kk, i);
        Kt[at] = ke;
        Kbt[at] = to_e<E>(sb * from_e<E>(ke));
        Vst[at] = to_e<E>(sv * from_e<E>(tile_elem<E, C, D>(vt, u, kk)));
      }
    }
  }
  __syncthreads();
  // K K^T (fp32); the products from here to the node tiles are taken with
  // swapped operands, so a lane writes four consecutive columns of one row
  for_tiles<C, C>([&](int m0, int n0) {
    const f32x4 acc = mm_kc<BF16, D, true>(Kr, LDD, Kr, LDD, m0, n0, f32x4{0.f, 0.f, 0.f, 0.f});
    *reinterpret_cast<f32x4*>(G + (m0 + tile_col()) * LF + n0 + tile_row0()) = acc;
  });
  __syncthreads();
  solve_blocked<C>(G, bet, Tm, X);   // in place: every entry of G is read before T is written over it
  // (T diag(beta))^T for the output kernel
  E* tb = static_cast<E*>(a.tb) + (bh * a.n_chunks + c) * (C * C);
  {
    constexpr int EPV = 16 / es, VR = C / EPV;
    for (int e = tid; e < C * VR; e += kGdnThreads) {
      const int s = e / VR, r0 = (e % VR) * EPV;
      float x[EPV];
#pragma unroll
      for (int kk = 0; kk < EPV; ++kk) x[kk] = Tm[(r0 + kk) * LF + s] * bet[s];
      reinterpret_cast<u32x4*>(tb)[e] = pack16<E>(x);
    }
  }
  gout = g;
  if (!full) return false;
  // U^T = (gated beta V)^T T^T over the scratch, then W^T = (beta K)^T T^T
  // over the (then dead) gated V tile
  for_tiles<D, C>([&](int m0, int n0) {
    const f32x4 acc = mm_sw<BF16, C, true, false, true>(Vst, 0, Tm, LF, m0, n0, f32x4{0.f, 0.f, 0.f, 0.f});
    store4<E>(Ut + swz<E, C>(m0 + tile_col(), n0 + tile_row0()), acc);
  });
  __syncthreads();
  for_tiles<D, C>([&](int m0, int n0) {
    const f32x4 acc = mm_sw<BF16, C, true, false, true>(Kbt, 0, Tm, LF, m0, n0, f32x4{0.f, 0.f, 0.f, 0.f});
    store4<E>(Wt + swz<E, C>(m0 + tile_col(), n0 + tile_row0()), acc);
  });
  __syncthreads();
  // P_c = K^T U and Psi_c = I - K^T W
  using PT = PrepTiles<D>;
#pragma unroll
  for (int u = 0; u < PT::NPW; ++u) {
    const int t = wave_id() + PT::NW * u;
    if (t < PT::NT) {
      const int m0 = (t / PT::TN) * 16, n0 = (t % PT::TN) * 16;
      P[u] = mm_sw<BF16, C, true, true>(Kt, 0, Ut, 0, m0, n0, f32x4{0.f, 0.f, 0.f, 0.f});
      const f32x4 acc = mm_sw<BF16, C, true, true>(Kt, 0, Wt, 0, m0, n0, f32x4{0.f, 0.f, 0.f, 0.f});
      const int col = n0 + tile_col(), row = m0 + tile_row0();
#pragma unroll
      for (int i = 0; i < 4; ++i) S[u][i] = (row + i == col ? 1.f : 0.f) - acc[i];
    }
  }
  return true;
}

// Node tiles held as in gdn_prep_chunk, stored transposed into node `node`.
template <bool BF16, int D>
__device__ __forceinline__ void store_node(const GdnArgs& a, int64_t node, const f32x4 (&P)[PrepTiles<D>::NPW],
                                           const f32x4 (&S)[PrepTiles<D>::NPW]) {
  using E = typename Elem<BF16>::T;
  using PT = PrepTiles<D>;
  E* pt = static_cast<E*>(a.pt) + node * (D * D);
  E* ps = static_cast<E*>(a.psit) + node * (D * D);
#pragma unroll
  for (int u = 0; u < PT::NPW; ++u) {
    const int t = wave_id() + PT::NW * u;
    if (t < PT::NT) {
      const int col = (t % PT::TN) * 16 + tile_col(), row = (t / PT::TN) * 16 + tile_row0();
      store4<E>(pt + col * D + row, P[u]);
      store4<E>(ps + col * D + row, S[u]);
    }
  }
}

// gdn_chunk_prep: one workgroup per (b,h, pair of chunks 2x, 2x+1).  The even
// chunk's level-0 node is stored (query chunk c reads the level-0 node of
// chunk c - 1 only for odd c); when both chunks are full, their level-1 node
// P = 2^(g_1) Psi_1 P_0 + P_1, Psi = Psi_1 Psi_0 is formed here from the
// register tiles, so odd level-0 nodes are never stored and the tree starts
// at level 2.
// bf16 tiles fit three prep workgroups per CU by LDS; the compiler is held
// to the 80 registers (six waves per SIMD) that allow it.
template <bool BF16>
constexpr int gdn_prep_min_waves() { return BF16 ? 6 : 1; }

template <bool BF16, int C, int D>
__global__ __launch_bounds__(kGdnThreads) __attribute__((amdgpu_waves_per_eu(gdn_prep_min_waves<BF16>(), 8)))
void gdn_chunk_prep(GdnArgs a) {
  using E = typename Elem<BF16>::T;
  using PT = PrepTiles<D>;
  constexpr int es = sizeof(E), LDD = gdn_lde(D, es), DD = D * D;
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t npair = (a.n_chunks + 1) / 2;
  const int64_t bh = blockIdx.x / npair, x = blockIdx.x % npair;
  const int64_t c0 = 2 * x, c1 = c0 + 1;
  f32x4 P0[PT::NPW], S0[PT::NPW], P1[PT::NPW], S1[PT::NPW];
  float g0 = 0.f, g1 = 0.f;
  const bool f0 = gdn_prep_chunk<BF16, C, D>(a, smem, bh, c0, P0, S0, g0);
  if (f0) {
    const int64_t node = a.lev_off[0] + bh * a.n_full + c0;
    store_node<BF16, D>(a, node, P0, S0);
    if (threadIdx.x == 0) a.gn[node] = g0;
  }
  if (c1 >= a.n_chunks) return;
  __syncthreads();   // the second chunk reuses the LDS
  const bool f1 = gdn_prep_chunk<BF16, C, D>(a, smem, bh, c1, P1, S1, g1);
  if (!f1) return;   // a full odd chunk implies a full even one
  __syncthreads();
  // Psi_1 row-major, P_0 and Psi_0 transposed (rows = d_v), over the dead tiles
  constexpr int TB = gdn_tile(D, D, es);
  E* A1 = reinterpret_cast<E*>(smem);
  E* B0 = reinterpret_cast<E*>(smem + TB);
  E* C0 = reinterpret_cast<E*>(smem + 2 * TB);
#pragma unroll
  for (int u = 0; u < PT::NPW; ++u) {
    const int t = wave_id() + PT::NW * u;
    if (t < PT::NT) {
      const int col = (t % PT::TN) * 16 + tile_col(), row = (t / PT::TN) * 16 + tile_row0();
#pragma unroll
      for (int i = 0; i < 4; ++i) A1[(row + i) * LDD + col] = to_e<E>(S1[u][i]);
      store4<E>(B0 + col * LDD + row, P0[u]);
      store4<E>(C0 + col * LDD + row, S0[u]);
    }
  }
  __syncthreads();
  const float s1 = __builtin_amdgcn_exp2f(g1);
  const int64_t node = a.lev_off[1] + bh * (a.n_full >> 1) + x;
  E* pt = static_cast<E*>(a.pt) + node * DD;
  E* ps = static_cast<E*>(a.psit) + node * DD;
#pragma unroll
  for (int u = 0; u < PT::NPW; ++u) {
    const int t = wave_id() + PT::NW * u;
    if (t < PT::NT) {
      const int m0 = (t / PT::TN) * 16, n0 = (t % PT::TN) * 16;
      const int col = n0 + tile_col(), row = m0 + tile_row0();
      const f32x4 ap = mm_kc<BF16, D>(A1, LDD, B0, LDD, m0, n0, f32x4{0.f, 0.f, 0.f, 0.f});
      const f32x4 as = mm_kc<BF16, D>(A1, LDD, C0, LDD, m0, n0, f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = fmaf(s1, ap[i], P1[u][i]);
      store4<E>(pt + col * D + row, o);
      store4<E>(ps + col * D + row, as);
    }
  }
  if (threadIdx.x == 0) a.gn[node] = g0 + g1;
}

// ---------------------------------------------------------------------------
// gdn_tree: one workgroup per block of 2^m chunks (m >= 2), merging the
// halves of level m - 1.
template <bool BF16, int D>
__global__ __launch_bounds__(kGdnThreads) void gdn_tree(GdnArgs a, int m) {
  using E = typename Elem<BF16>::T;
  constexpr int es = sizeof(E), LDD = gdn_lde(D, es), DD = D * D;
  extern __shared__ __align__(16) unsigned char smem[];
  E* PsiR = reinterpret_cast<E*>(smem);   // Psi of the right half, row-major
  const int64_t nm = a.n_full >> m, np = a.n_full >> (m - 1);
  const int64_t bh = blockIdx.x / nm, x = blockIdx.x % nm;
  const int64_t iL = a.lev_off[m - 1] + bh * np + 2 * x, iR = iL + 1;
  const int64_t io = a.lev_off[m] + bh * nm + x;
  const E* pt = static_cast<const E*>(a.pt);
  const E* ps = static_cast<const E*>(a.psit);
  using TV = TileVec<D, D, es>;
  const TV pr = load_tile<D, D>(ps + iR * DD, D);
  // each wave owns column strips (of P or of Psi): their B operands, taken
  // from the left half in global memory, are loaded once, before the wait
  constexpr int TN = D / 16, NJ = 2 * TN, NW = kGdnThreads / 64, JPW = (NJ + NW - 1) / NW;
  BStrip<BF16, D> bs[JPW];
#pragma unroll
  for (int u = 0; u < JPW; ++u) {
    const int j = wave_id() + NW * u;
    if (j < NJ) bs[u] = load_strip<BF16, D>((j >= TN ? ps : pt) + iL * DD, D, 16 * (j % TN));
  }
  // and the state of the right half at this lane's outputs (P strips only)
  f32x4 pR[JPW][D / 16];
#pragma unroll
  for (int u = 0; u < JPW; ++u) {
    const int j = wave_id() + NW * u;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      pR[u][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j < TN) pR[u][mb] = load4<E>(pt + iR * DD + (16 * j + tile_col()) * D + 16 * mb + tile_row0());
    }
  }
#pragma unroll
  for (int u = 0; u < TV::VPT; ++u) {
    const int e = threadIdx.x + kGdnThreads * u;
    if (e < TV::NV) {
      const int i = tile_row<D, TV::VPR>(e), j0 = tile_vcol<D, TV::VPR>(e) * TV::EPV;
#pragma unroll
      for (int kk = 0; kk < TV::EPV; ++kk) PsiR[(j0 + kk) * LDD + i] = tile_elem<E, D, D>(pr, u, kk);
    }
  }
  const float gR = a.gn[iR];
  const float sR = __builtin_amdgcn_exp2f(gR);
  __syncthreads();
  E* pto = static_cast<E*>(a.pt) + io * DD;
  E* pso = static_cast<E*>(a.psit) + io * DD;
  // P = 2^gR Psi_R P_L + P_R ; Psi = Psi_R Psi_L (both stored transposed)
#pragma unroll
  for (int u = 0; u < JPW; ++u) {
    const int j = wave_id() + NW * u;
    if (j < NJ) {
      const bool isp = j >= TN;
      const int col = 16 * (j % TN) + tile_col();
#pragma unroll
      for (int m0 = 0; m0 < D; m0 += 16) {
        const f32x4 acc = mm_strip<BF16, D>(PsiR, LDD, bs[u], m0, f32x4{0.f, 0.f, 0.f, 0.f});
        const int row = m0 + tile_row0();
        f32x4 o = acc;
        if (!isp) {
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = fmaf(sR, acc[i], pR[u][m0 / 16][i]);
        }
        store4<E>((isp ? pso : pto) + col * D + row, o);
      }
    }
  }
  if (threadIdx.x == 0) a.gn[io] = a.gn[iL] + gR;
}

// ---------------------------------------------------------------------------
// gdn_chunk_output: one workgroup of four waves per (b,h, chunk).  LDS holds
// Q (then the carried queries), K (then Ahat), V (then the masked tile P),
// tril(Q K^T) (then the second carried-query buffer), the chunk's lambda rows
// in the layer dtype, its gate scan and betas: 38 KB at C = d = 64 in bf16,
// so four workgroups fit a CU.  Wave w owns the 16-column strip 16 (w % TN)
// of every product and keeps its B operands in registers: the K and V strips
// taken along the tokens before those tiles are overwritten, (T diag(beta))^T
// and the bucket nodes straight from global memory.
// bf16 tiles fit four workgroups per CU by LDS; the compiler is held to the
// 128 registers that allow it (no spills).  fp32 tiles are larger and are
// left unconstrained.
template <bool BF16>
constexpr int gdn_out_min_waves() { return BF16 ? 4 : 1; }

template <bool BF16, int C, int D>
__global__ __launch_bounds__(kGdnOutThreads) __attribute__((amdgpu_waves_per_eu(gdn_out_min_waves<BF16>(), 8)))
void gdn_chunk_output(GdnArgs a) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  constexpr int NT = kGdnOutThreads, NW = NT / 64;
  constexpr int es = sizeof(E);
  constexpr int LDD = gdn_lde(D, es), LDC = gdn_lde(C, es);
  constexpr int TNC = C / 16, TND = D / 16, RB = C / 16;
  constexpr int OCC = (RB * TNC + NW - 1) / NW, OCD = (RB * TND + NW - 1) / NW;
  const GdnOutLds LY = gdn_out_lds(C, D, es, a.L);
  extern __shared__ __align__(16) unsigned char smem[];
  E* Ql = reinterpret_cast<E*>(smem + LY.q);
  E* Kl = reinterpret_cast<E*>(smem + LY.k);
  E* Al = Kl;                                      // Ahat, over K once its strips are taken
  E* Vl = reinterpret_cast<E*>(smem + LY.v);
  E* Pl = Vl;                                      // P, over V once its strip is taken
  E* Sl = reinterpret_cast<E*>(smem + LY.s);
  E* lam = reinterpret_cast<E*>(smem + LY.lam);
  float* b2 = reinterpret_cast<float*>(smem + LY.b2);
  float* bet = reinterpret_cast<float*>(smem + LY.beta);
  const int L = a.L;
  const int64_t bh = blockIdx.x / a.n_chunks, c = blockIdx.x % a.n_chunks;
  const int64_t t0 = c * C;
  const int nv = (int)((a.T - t0) < C ? (a.T - t0) : C);
  const int tid = threadIdx.x, w = wave_id();
  const int n0c = 16 * (w % TNC), n0d = 16 * (w % TND);
  const int64_t row0 = bh * a.T + t0;
  using TV = TileVec<C, D, es, NT>;
  const TV tq = load_tile_c<C, D, NT>(static_cast<const E*>(a.q) + row0 * D, nv);
  const TV tk = load_tile_c<C, D, NT>(static_cast<const E*>(a.k) + row0 * D, nv);
  const TV tvv = load_tile_c<C, D, NT>(static_cast<const E*>(a.v) + row0 * D, nv);
  constexpr int LPT = (C * kMaxLevels + NT - 1) / NT;
  float lv[LPT];
  const float* lp = a.lam + row0 * L;
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int e = tid + NT * u;
    lv[u] = e < nv * L ? lp[e] : 0.f;
  }
  // the B strips this wave needs from global memory, issued early: the
  // columns of (T diag(beta))^T for Ahat, and the first two bucket nodes'
  // states and transitions
  const E* tbp = static_cast<const E*>(a.tb) + (bh * a.n_chunks + c) * (C * C);
  const BStrip<BF16, C> tbs = load_strip<BF16, C>(tbp, C, n0c);
  const E* ptb = static_cast<const E*>(a.pt);
  const E* psb = static_cast<const E*>(a.psit);
  const int64_t nf = a.n_full;
  auto next_bit = [&](int m) -> int {   // next set bit of c above m, or -1
    const int64_t up = m < 0 ? c : (c >> (m + 1));
    return up == 0 ? -1 : (m + 1 + __builtin_ctzll((unsigned long long)up));
  };
  auto load_node = [&](int m, BStrip<BF16, D>& P, BStrip<BF16, D>& S) {
    const int64_t node = a.lev_off[m] + bh * (nf >> m) + (c >> m) - 1;
    P = load_strip<BF16, D>(ptb + node * (D * D), D, n0d);
    if (next_bit(m) >= 0) S = load_strip<BF16, D>(psb + node * (D * D), D, n0d);
  };
  BStrip<BF16, D> pf{}, sf{}, pn{}, sn{};
  const int mfirst = next_bit(-1);
  if (mfirst >= 0) {
    load_node(mfirst, pf, sf);
    const int msec = next_bit(mfirst);
    if (msec >= 0) load_node(msec, pn, sn);
  }
  if (w == 0) gdn_gate_scan<C>(a.log_a + bh * a.T, a.beta + bh * a.T, t0, nv, b2, bet);
#pragma unroll
  for (int u = 0; u < TV::VPT; ++u) {
    const int e = tid + NT * u;
    if (e < TV::NV) {
      const int i = tile_row_c<C, TV::VPR>(e), j0 = tile_vcol_c<C, TV::VPR>(e) * TV::EPV;
      *reinterpret_cast<u32x4*>(Ql + i * LDD + j0) = tq.v[u];
      *reinterpret_cast<u32x4*>(Kl + i * LDD + j0) = tk.v[u];
      *reinterpret_cast<u32x4*>(Vl + i * LDD + j0) = tvv.v[u];
    }
  }
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int e = tid + NT * u;
    if (e < C * L) lam[e] = to_e<E>(lv[u]);
  }
  __syncthreads();
  // the K and V strips, then tril(Q K^T).  Every product from here on is
  // taken transposed: lane l holds row m0 + l % 16 of the result at the four
  // consecutive columns 16 (strip) + 4 (l / 16) + i.
  const BStrip<BF16, D> ks = load_strip<BF16, D>(Kl, LDD, n0c);
  const BStrip<BF16, C> kts = load_strip_t<BF16, C>(Kl, LDD, n0d);
  const BStrip<BF16, C> vts = load_strip_t<BF16, C>(Vl, LDD, n0d);
  const int orow = tile_col(), ocol = n0d + tile_row0(), ccol = n0c + tile_row0();
#pragma unroll
  for (int u = 0; u < OCC; ++u) {
    const int t = w + NW * u;
    if (t < RB * TNC) {
      const int m0 = (t / TNC) * 16, row = m0 + orow;
      const f32x4 acc = n0c > m0 ? f32x4{0.f, 0.f, 0.f, 0.f}   // above the diagonal
                                 : mm_strip_t<BF16, D>(Ql, LDD, ks, m0, f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 sv;
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = ccol + i <= row ? acc[i] : 0.f;
      store4<E>(Sl + row * LDC + ccol, sv);
    }
  }
  __syncthreads();
  // Ahat = tril(Q K^T) T diag(beta), and from it the masked intra tile P:
  // lambda of the level and the gate ratio
#pragma unroll
  for (int u = 0; u < OCC; ++u) {
    const int t = w + NW * u;
    if (t < RB * TNC) {
      const int m0 = (t / TNC) * 16, tr = m0 + orow;
      // tril(Q K^T) rows m0.. vanish past key m0 + 15 and the columns n0c.. of
      // the lower triangular T diag(beta) before key n0c
      const f32x4 acc = mm_strip_t<BF16, C>(Sl, LDC, tbs, m0, f32x4{0.f, 0.f, 0.f, 0.f}, n0c, m0 + 16);
      store4<E>(Al + tr * LDC + ccol, acc);
      const float b2r = b2[tr];
      const f32x4 b2c = *reinterpret_cast<const f32x4*>(b2 + ccol);
      f32x4 pv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = ccol + i;
        pv[i] = 0.f;
        if (col <= tr && tr < nv)
          pv[i] = acc[i] * from_e<E>(lam[tr * L + fenwick_level_local((unsigned)tr, (unsigned)col)]) *
                  __builtin_amdgcn_exp2f(b2r - b2c[i]);
      }
      store4<E>(Pl + tr * LDC + ccol, pv);
    }
  }
  __syncthreads();
  // carried queries Q' = Q - Ahat K (in place) and O = P V in registers
  f32x4 o[OCD];
#pragma unroll
  for (int u = 0; u < OCD; ++u) {
    const int t = w + NW * u;
    o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t < RB * TND) {
      const int m0 = (t / TND) * 16;
      // Ahat and P are lower triangular: rows m0.. vanish past key m0 + 15
      const f32x4 acc = mm_strip_t<BF16, C>(Al, LDC, kts, m0, f32x4{0.f, 0.f, 0.f, 0.f}, 0, m0 + 16);
      E* qe = Ql + (m0 + orow) * LDD + ocol;
      const f32x4 q4 = load4<E>(qe);
      store4<E>(qe, f32x4{q4[0] - acc[0], q4[1] - acc[1], q4[2] - acc[2], q4[3] - acc[3]});
      o[u] = mm_strip_t<BF16, C>(Pl, LDC, vts, m0, o[u], 0, m0 + 16);
    }
  }
  __syncthreads();   // the carried queries are complete
  // bucket nodes of the set bits of c, most recent first; the node two levels
  // ahead is loaded while this one is used.  Row weights are
  // lambda * 2^(b_t) * 2^(G): the per-row gate is formed once (both exponents
  // are <= 0, so the split only moves underflow below 2^-126)
  constexpr int log2C = gdn_clog2(C);
  float gam[OCD];
#pragma unroll
  for (int u = 0; u < OCD; ++u) {
    const int t = w + NW * u;
    gam[u] = t < RB * TND ? __builtin_amdgcn_exp2f(b2[(t / TND) * 16 + orow]) : 0.f;
  }
  E* cur = Ql;
  E* nxt = Sl;
  float Gs = 0.f;
  for (int m = mfirst; m >= 0; m = next_bit(m)) {
    const int64_t node = a.lev_off[m] + bh * (nf >> m) + (c >> m) - 1;
    const int lev = log2C + 1 + m;
    const int64_t up = c >> (m + 1);
    BStrip<BF16, D> pn2{}, sn2{};
    const int m3 = next_bit(next_bit(m) < 0 ? 62 : next_bit(m));
    if (m3 >= 0) load_node(m3, pn2, sn2);
    const float sg = __builtin_amdgcn_exp2f(Gs);
#pragma unroll
    for (int u = 0; u < OCD; ++u) {
      const int t = w + NW * u;
      if (t < RB * TND) {
        const int m0 = (t / TND) * 16;
        const f32x4 y = mm_strip_t<BF16, D>(cur, LDD, pf, m0, f32x4{0.f, 0.f, 0.f, 0.f});
        const float wr = from_e<E>(lam[(m0 + orow) * L + lev]) * gam[u] * sg;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[u][i] = fmaf(wr, y[i], o[u][i]);
      }
    }
    if (up != 0) {   // an older node follows: carry the queries through this block
#pragma unroll
      for (int u = 0; u < OCD; ++u) {
        const int t = w + NW * u;
        if (t < RB * TND) {
          const int m0 = (t / TND) * 16;
          store4<E>(nxt + (m0 + orow) * LDD + ocol, mm_strip_t<BF16, D>(cur, LDD, sf, m0, f32x4{0.f, 0.f, 0.f, 0.f}));
        }
      }
      Gs += a.gn[node];
      __syncthreads();
      E* sw = cur;
      cur = nxt;
      nxt = sw;
      pf = pn;
      sf = sn;
      pn = pn2;
      sn = sn2;
    }
  }
  E* op = static_cast<E*>(a.out) + row0 * D;
#pragma unroll
  for (int u = 0; u < OCD; ++u) {
    const int t = w + NW * u;
    if (t < RB * TND) {
      const int row = (t / TND) * 16 + orow;
      if (row < nv) store4<E>(op + row * D + ocol, o[u]);
    }
  }
}

// ---------------------------------------------------------------------------
template <bool BF16, int C, int D>
int launch_gdn_impl(const GdnPlan& p, const GdnArgs& a, hipStream_t s) {
  bool ok = hipFuncSetAttribute((const void*)gdn_chunk_prep<BF16, C, D>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_prep) == hipSuccess;
  if (!ok) return kEHIP;
  hipLaunchKernelGGL((gdn_chunk_prep<BF16, C, D>), dim3((unsigned)(p.BH * ((p.n_chunks + 1) / 2))),
                     dim3(kGdnThreads), p.lds_prep, s, a);
  ok = hipGetLastError() == hipSuccess;
  for (int m = 2; m < p.n_tree && ok; ++m) {   // level 1 comes from the prep kernel
    hipLaunchKernelGGL((gdn_tree<BF16, D>), dim3((unsigned)(p.BH * (p.n_full >> m))), dim3(kGdnThreads),
                       p.lds_tree, s, a, m);
    ok = hipGetLastError() == hipSuccess;
  }
  ok = ok && hipFuncSetAttribute((const void*)gdn_chunk_output<BF16, C, D>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_out) == hipSuccess;
  if (!ok) return kEHIP;
  hipLaunchKernelGGL((gdn_chunk_output<BF16, C, D>), dim3((unsigned)(p.BH * p.n_chunks)), dim3(kGdnOutThreads),
                     p.lds_out, s, a);
  ok = hipGetLastError() == hipSuccess;
  return ok ? kOK : kEHIP;
}

template <bool BF16>
int launch_gdn_dtype(const GdnPlan& p, const GdnArgs& a, hipStream_t s) {
#define LA_CASE(CC, DD) \
  if (p.C == CC && p.D == DD) return launch_gdn_impl<BF16, CC, DD>(p, a, s);
  LA_CASE(16, 16) LA_CASE(16, 32) LA_CASE(16, 64)
  LA_CASE(32, 16) LA_CASE(32, 32) LA_CASE(32, 64)
  LA_CASE(64, 16) LA_CASE(64, 32) LA_CASE(64, 64)
#undef LA_CASE
  return kESHAPE;
}

}  // namespace la
