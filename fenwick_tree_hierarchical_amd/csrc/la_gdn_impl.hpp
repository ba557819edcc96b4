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
// Kernels (each workgroup 4 waves; all tiles staged in LDS as fp32; in bf16
// mode every matrix-core operand is rounded to bf16, fp32 accumulation):
//   gdn_chunk_prep    per full chunk: P_c, Psi_c, g_c (the tree's level 0)
//   gdn_tree          per block of 2^m chunks: the merge of its two halves
//   gdn_chunk_output  per chunk: the intra tile, the carried queries and the
//                     level contractions; writes the output.
#pragma once

#include "la_device.hpp"
#include "la_gdn_plan.hpp"

namespace la {

struct GdnArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_a;
  const float* beta;
  const float* lam;
  void* out;
  float* pt;     // [n_nodes][D][D] block states, (d_v, d_k) order
  float* psit;   // [n_nodes][D][D] block transitions without gates, transposed
  float* gn;     // [n_nodes] block log2 gate totals
  int64_t T;
  int64_t n_chunks;
  int64_t n_full;
  int L;
  int64_t lev_off[kGdnMaxTree];
};

// acc += A[m0:m0+16, 0:K] * B[0:K, n0:n0+16] on the matrix cores.
// AKC: A is stored A[m * lda + k] (else A[k * lda + m]);
// BKC: B is stored B[n * ldb + k] (else B[k * ldb + n]).
// Lane l supplies row/column l % 16 and the k-slice l / 16 of its operands;
// the result holds, in lane l, rows 4 (l / 16) + i of column l % 16.
template <bool BF16, bool AKC, bool BKC, int K>
__device__ __forceinline__ f32x4 mm_tile(const float* A, int lda, const float* B, int ldb, int m0, int n0,
                                         f32x4 acc) {
  const int lane = lane_id(), r = lane & 15, kq = lane >> 4;
  if constexpr (BF16) {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
      const int kk = k0 + 8 * kq;
      bf16x8 fa, fb;
      if (kk < K) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          fa[i] = (__bf16)(AKC ? A[(m0 + r) * lda + kk + i] : A[(kk + i) * lda + m0 + r]);
          fb[i] = (__bf16)(BKC ? B[(n0 + r) * ldb + kk + i] : B[(kk + i) * ldb + n0 + r]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          fa[i] = (__bf16)0.f;
          fb[i] = (__bf16)0.f;
        }
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4) {
      const int kk = k0 + kq;
      const float fa = AKC ? A[(m0 + r) * lda + kk] : A[kk * lda + m0 + r];
      const float fb = BKC ? B[(n0 + r) * ldb + kk] : B[kk * ldb + n0 + r];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa, fb, acc, 0, 0, 0);
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

constexpr int gdn_clog2(int x) { return x <= 1 ? 0 : 1 + gdn_clog2(x >> 1); }

__device__ __forceinline__ int tile_row0() { return 4 * (lane_id() >> 4); }
__device__ __forceinline__ int tile_col() { return lane_id() & 15; }

// T^T for T = (I + L)^-1, L[i][m] = beta_i G[i][m] for m < i (unit lower
// triangular), by forward substitution: lane j solves column j.  One wave.
template <int C>
__device__ __forceinline__ void solve_unit_lower(const float* G, int ld, const float* beta, float* Tt) {
  const int j = lane_id();
  float x[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;   // four chains hide the FMA latency
#pragma unroll
    for (int m = 0; m + 3 < i; m += 4) {
      p0 = fmaf(G[i * ld + m], x[m], p0);
      p1 = fmaf(G[i * ld + m + 1], x[m + 1], p1);
      p2 = fmaf(G[i * ld + m + 2], x[m + 2], p2);
      p3 = fmaf(G[i * ld + m + 3], x[m + 3], p3);
    }
#pragma unroll
    for (int m = i & ~3; m < i; ++m) p0 = fmaf(G[i * ld + m], x[m], p0);
    x[i] = (i == j ? 1.f : 0.f) - beta[i] * ((p0 + p1) + (p2 + p3));
  }
  if (j < C) {
#pragma unroll
    for (int i = 0; i < C; ++i) Tt[j * ld + i] = x[i];
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
// gdn_chunk_prep: one workgroup per (b,h, full chunk).  Level-0 nodes.
template <bool BF16, int C, int D>
__global__ __launch_bounds__(kGdnThreads) void gdn_chunk_prep(GdnArgs a) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  constexpr int LD = gdn_ld(C, D);
  constexpr GdnPrepLds LY = gdn_prep_lds(C, D);
  extern __shared__ __align__(16) unsigned char smem[];
  float* Kl = reinterpret_cast<float*>(smem + LY.k);
  float* Vs = reinterpret_cast<float*>(smem + LY.vs);
  float* Kb = reinterpret_cast<float*>(smem + LY.kb);
  float* Gm = reinterpret_cast<float*>(smem + LY.g);
  float* Tt = reinterpret_cast<float*>(smem + LY.tt);
  float* Wl = reinterpret_cast<float*>(smem + LY.w);
  float* b2 = reinterpret_cast<float*>(smem + LY.b2);
  float* bet = reinterpret_cast<float*>(smem + LY.beta);
  const int64_t nf = a.n_full;
  const int64_t bh = blockIdx.x / nf, c = blockIdx.x % nf;
  const int64_t t0 = c * C;
  const int tid = threadIdx.x;
  if (wave_id() == 0) gdn_gate_scan<C>(a.log_a + bh * a.T, a.beta + bh * a.T, t0, C, b2, bet);
  __syncthreads();
  const float g = b2[C - 1];
  const E* kp = static_cast<const E*>(a.k) + (bh * a.T + t0) * D;
  const E* vp = static_cast<const E*>(a.v) + (bh * a.T + t0) * D;
  for (int e = tid; e < C * D; e += kGdnThreads) {
    const int i = e / D, j = e % D;
    const float kv = EL::to_f32(kp[e]), vv = EL::to_f32(vp[e]);
    Kl[i * LD + j] = kv;
    Kb[i * LD + j] = bet[i] * kv;
    Vs[i * LD + j] = bet[i] * exp2f(g - b2[i]) * vv;
  }
  __syncthreads();
  // K K^T
  for_tiles<C, C>([&](int m0, int n0) {
    const f32x4 acc = mm_tile<BF16, true, true, D>(Kl, LD, Kl, LD, m0, n0, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int i = 0; i < 4; ++i) Gm[(m0 + tile_row0() + i) * LD + n0 + tile_col()] = acc[i];
  });
  __syncthreads();
  if (wave_id() == 0) solve_unit_lower<C>(Gm, LD, bet, Tt);
  __syncthreads();
  // U = T Vs (over K K^T) and W = T Kb
  for_tiles<C, 2 * D>([&](int m0, int n0) {
    const bool isw = n0 >= D;
    const int nn = isw ? n0 - D : n0;
    const f32x4 acc =
        mm_tile<BF16, false, false, C>(Tt, LD, isw ? Kb : Vs, LD, m0, nn, f32x4{0.f, 0.f, 0.f, 0.f});
    float* dst = isw ? Wl : Gm;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(m0 + tile_row0() + i) * LD + nn + tile_col()] = acc[i];
  });
  __syncthreads();
  // P_c = K^T U and Psi_c = I - K^T W, stored transposed
  const int64_t node = a.lev_off[0] + bh * nf + c;
  float* pt = a.pt + node * (D * D);
  float* ps = a.psit + node * (D * D);
  for_tiles<D, 2 * D>([&](int m0, int n0) {
    const bool isw = n0 >= D;
    const int nn = isw ? n0 - D : n0;
    const f32x4 acc =
        mm_tile<BF16, false, false, C>(Kl, LD, isw ? Wl : Gm, LD, m0, nn, f32x4{0.f, 0.f, 0.f, 0.f});
    const int col = nn + tile_col(), row = m0 + tile_row0();
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = isw ? ((row + i == col ? 1.f : 0.f) - acc[i]) : acc[i];
    *reinterpret_cast<f32x4*>((isw ? ps : pt) + col * D + row) = o;
  });
  if (tid == 0) a.gn[node] = g;
}

// ---------------------------------------------------------------------------
// gdn_tree: one workgroup per block of 2^m chunks (m >= 1), merging the
// halves of level m - 1.
template <bool BF16, int D>
__global__ __launch_bounds__(kGdnThreads) void gdn_tree(GdnArgs a, int m) {
  const int64_t nm = a.n_full >> m, np = a.n_full >> (m - 1);
  const int64_t bh = blockIdx.x / nm, x = blockIdx.x % nm;
  const int64_t iL = a.lev_off[m - 1] + bh * np + 2 * x, iR = iL + 1;
  const int64_t io = a.lev_off[m] + bh * nm + x;
  constexpr int DD = D * D;
  const float gR = a.gn[iR];
  const float sR = exp2f(gR);
  const float* psR = a.psit + iR * DD;
  for_tiles<D, 2 * D>([&](int m0, int n0) {
    const bool isp = n0 >= D;
    const int nn = isp ? n0 - D : n0;
    // P = 2^gR Psi_R P_L + P_R ; Psi = Psi_R Psi_L
    const float* Bop = isp ? a.psit + iL * DD : a.pt + iL * DD;
    const f32x4 acc = mm_tile<BF16, false, true, D>(psR, D, Bop, D, m0, nn, f32x4{0.f, 0.f, 0.f, 0.f});
    const int col = nn + tile_col(), row = m0 + tile_row0();
    f32x4 o;
    if (isp) {
      o = acc;
    } else {
      const f32x4 pr = *reinterpret_cast<const f32x4*>(a.pt + iR * DD + col * D + row);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = fmaf(sR, acc[i], pr[i]);
    }
    *reinterpret_cast<f32x4*>((isp ? a.psit : a.pt) + io * DD + col * D + row) = o;
  });
  if (threadIdx.x == 0) a.gn[io] = a.gn[iL] + gR;
}

// ---------------------------------------------------------------------------
// gdn_chunk_output: one workgroup per (b,h, chunk).
template <bool BF16, int C, int D>
__global__ __launch_bounds__(kGdnThreads) void gdn_chunk_output(GdnArgs a) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  constexpr int LD = gdn_ld(C, D);
  const GdnOutLds LY = gdn_out_lds(C, D, a.L);
  extern __shared__ __align__(16) unsigned char smem[];
  float* Ql = reinterpret_cast<float*>(smem + LY.q);
  float* Kl = reinterpret_cast<float*>(smem + LY.k);
  float* Vl = reinterpret_cast<float*>(smem + LY.v);
  float* Sl = reinterpret_cast<float*>(smem + LY.s);
  float* Al = reinterpret_cast<float*>(smem + LY.a);
  float* Tt = reinterpret_cast<float*>(smem + LY.tt);
  float* lam = reinterpret_cast<float*>(smem + LY.lam);
  float* b2 = reinterpret_cast<float*>(smem + LY.b2);
  float* bet = reinterpret_cast<float*>(smem + LY.beta);
  const int L = a.L;
  const int64_t bh = blockIdx.x / a.n_chunks, c = blockIdx.x % a.n_chunks;
  const int64_t t0 = c * C;
  const int nv = (int)((a.T - t0) < C ? (a.T - t0) : C);
  const int tid = threadIdx.x;
  if (wave_id() == 0) gdn_gate_scan<C>(a.log_a + bh * a.T, a.beta + bh * a.T, t0, nv, b2, bet);
  const int64_t row0 = bh * a.T + t0;
  const E* qp = static_cast<const E*>(a.q) + row0 * D;
  const E* kp = static_cast<const E*>(a.k) + row0 * D;
  const E* vp = static_cast<const E*>(a.v) + row0 * D;
  for (int e = tid; e < C * D; e += kGdnThreads) {
    const int i = e / D, j = e % D;
    const bool ok = i < nv;
    Ql[i * LD + j] = ok ? EL::to_f32(qp[e]) : 0.f;
    Kl[i * LD + j] = ok ? EL::to_f32(kp[e]) : 0.f;
    Vl[i * LD + j] = ok ? EL::to_f32(vp[e]) : 0.f;
  }
  const float* lp = a.lam + row0 * L;
  for (int e = tid; e < C * L; e += kGdnThreads) lam[e] = e < nv * L ? lp[e] : 0.f;
  __syncthreads();
  // tril(Q K^T) and K K^T
  for_tiles<C, 2 * C>([&](int m0, int n0) {
    const bool isg = n0 >= C;
    const int nn = isg ? n0 - C : n0;
    const float* Aop = isg ? Kl : Ql;
    const f32x4 acc = mm_tile<BF16, true, true, D>(Aop, LD, Kl, LD, m0, nn, f32x4{0.f, 0.f, 0.f, 0.f});
    const int col = nn + tile_col(), row = m0 + tile_row0();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (isg) Al[(row + i) * LD + col] = acc[i];
      else Sl[(row + i) * LD + col] = col <= row + i ? acc[i] : 0.f;
    }
  });
  __syncthreads();
  if (wave_id() == 0) solve_unit_lower<C>(Al, LD, bet, Tt);
  __syncthreads();
  // Ahat = tril(Q K^T) T diag(beta), over K K^T
  for_tiles<C, C>([&](int m0, int n0) {
    const f32x4 acc = mm_tile<BF16, true, true, C>(Sl, LD, Tt, LD, m0, n0, f32x4{0.f, 0.f, 0.f, 0.f});
    const int col = n0 + tile_col(), row = m0 + tile_row0();
    const float bcol = bet[col];
#pragma unroll
    for (int i = 0; i < 4; ++i) Al[(row + i) * LD + col] = acc[i] * bcol;
  });
  __syncthreads();
  // carried queries Q' = Q - Ahat K, in place
  for_tiles<C, D>([&](int m0, int n0) {
    const f32x4 acc = mm_tile<BF16, true, false, C>(Al, LD, Kl, LD, m0, n0, f32x4{0.f, 0.f, 0.f, 0.f});
    const int col = n0 + tile_col(), row = m0 + tile_row0();
#pragma unroll
    for (int i = 0; i < 4; ++i) Ql[(row + i) * LD + col] -= acc[i];
  });
  __syncthreads();
  // the masked intra tile: lambda of the level and the gate ratio
  for (int e = tid; e < C * C; e += kGdnThreads) {
    const int i = e / C, j = e % C;
    float p = 0.f;
    if (j <= i && i < nv) p = Al[i * LD + j] * lam[i * L + fenwick_level_local((unsigned)i, (unsigned)j)] * exp2f(b2[i] - b2[j]);
    Al[i * LD + j] = p;
  }
  __syncthreads();
  // O = P V, each wave keeping its output tiles in registers
  constexpr int TN = D / 16, OT = (C / 16) * TN, NW = kGdnThreads / 64, OPW = (OT + NW - 1) / NW;
  f32x4 o[OPW];
#pragma unroll
  for (int u = 0; u < OPW; ++u) {
    const int t = wave_id() + NW * u;
    o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t < OT) o[u] = mm_tile<BF16, true, false, C>(Al, LD, Vl, LD, (t / TN) * 16, (t % TN) * 16, o[u]);
  }
  // bucket nodes of the set bits of c, most recent first
  constexpr int log2C = gdn_clog2(C);
  float* cur = Ql;
  float* nxt = Sl;
  float G = 0.f;
  const int64_t nf = a.n_full;
  for (int m = 0; (c >> m) != 0; ++m) {
    if (!((c >> m) & 1)) continue;
    const int64_t node = a.lev_off[m] + bh * (nf >> m) + (c >> m) - 1;
    const float* P = a.pt + node * (D * D);
    const int lev = log2C + 1 + m;
#pragma unroll
    for (int u = 0; u < OPW; ++u) {
      const int t = wave_id() + NW * u;
      if (t < OT) {
        const int m0 = (t / TN) * 16, n0 = (t % TN) * 16;
        const f32x4 y = mm_tile<BF16, true, true, D>(cur, LD, P, D, m0, n0, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m0 + tile_row0() + i;
          o[u][i] = fmaf(lam[row * L + lev] * exp2f(b2[row] + G), y[i], o[u][i]);
        }
      }
    }
    if ((c >> (m + 1)) != 0) {   // an older node follows: carry the queries through this block
      const float* Ps = a.psit + node * (D * D);
      for_tiles<C, D>([&](int m0, int n0) {
        const f32x4 acc = mm_tile<BF16, true, true, D>(cur, LD, Ps, D, m0, n0, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) nxt[(m0 + tile_row0() + i) * LD + n0 + tile_col()] = acc[i];
      });
      G += a.gn[node];
      __syncthreads();
      float* sw = cur;
      cur = nxt;
      nxt = sw;
    }
  }
  E* op = static_cast<E*>(a.out) + row0 * D;
#pragma unroll
  for (int u = 0; u < OPW; ++u) {
    const int t = wave_id() + NW * u;
    if (t < OT) {
      const int m0 = (t / TN) * 16, n0 = (t % TN) * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + tile_row0() + i;
        if (row < nv) op[row * D + n0 + tile_col()] = EL::from_f32(o[u][i]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <bool BF16, int C, int D>
int launch_gdn_impl(const GdnPlan& p, const GdnArgs& a, hipStream_t s) {
  bool ok = true;
  if (p.n_full >= 1) {
    ok = ok && hipFuncSetAttribute((const void*)gdn_chunk_prep<BF16, C, D>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_prep) == hipSuccess;
    if (!ok) return kEHIP;
    hipLaunchKernelGGL((gdn_chunk_prep<BF16, C, D>), dim3((unsigned)(p.BH * p.n_full)), dim3(kGdnThreads),
                       p.lds_prep, s, a);
    ok = ok && hipGetLastError() == hipSuccess;
    for (int m = 1; m < p.n_tree && ok; ++m) {
      hipLaunchKernelGGL((gdn_tree<BF16, D>), dim3((unsigned)(p.BH * (p.n_full >> m))), dim3(kGdnThreads), 0, s,
                         a, m);
      ok = ok && hipGetLastError() == hipSuccess;
    }
  }
  ok = ok && hipFuncSetAttribute((const void*)gdn_chunk_output<BF16, C, D>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_out) == hipSuccess;
  if (!ok) return kEHIP;
  hipLaunchKernelGGL((gdn_chunk_output<BF16, C, D>), dim3((unsigned)(p.BH * p.n_chunks)), dim3(kGdnThreads),
                     p.lds_out, s, a);
  ok = ok && hipGetLastError() == hipSuccess;
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
