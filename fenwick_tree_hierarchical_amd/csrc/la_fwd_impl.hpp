// Chunkwise-parallel forward of log-linear Mamba-2 attention for gfx950.
//
// "Log-Linear Attention" (Italian summary, technical section 2, item 3;
// Spanish summary, technical section 2, "Algoritmo de entrenamiento"): the
// sequence is cut into chunks; pairs inside a chunk are formed densely and
// pairs across chunks go through low-rank chunk states combined along the
// Fenwick levels.  With chunks of C = 2^c tokens the level of a pair splits
// exactly (0-based t, s):
//   same chunk       l = fenwick_level_local(t mod C, s mod C)   in [0, c]
//   different chunks l = c + 1 + msb(chunk_t xor chunk_s)
// so the levels above c form a Fenwick tree over chunks.  This file nests
// that once more: a workgroup owns a group of G = 2^g consecutive chunks and
//   * forms the C x C masked score tile of each chunk on the matrix cores
//     (levels 0..c),
//   * carries the chunk-level Fenwick buckets of its group (levels
//     c+1..c+g) in LDS with the binary-counter merge of the decode
//     recurrence, applied to whole chunks,
//   * reads the group-level buckets (levels > c+g) as precomputed nodes.
// Three kernels:
//   fwd_group_state  A_gamma = sum_{s in group} decay(s -> group end) k_s v_s^T
//   fwd_group_tree   per (b,h), a binary-counter walk over groups that writes
//                    node[e] = the Fenwick bucket ending at group e
//                    (2^ctz(e+1) groups), decayed to the end of group e, and the
//                    float64 prefix sums of the group gate totals
//   fwd_output       everything else, and the output.
// Gates are carried in log2 units (log_a * log2 e); every exponent that is
// applied is <= 0.  Chunk-local sums are float32, sums across groups float64.
#pragma once

#include "la_device.hpp"
#include "la_plan.hpp"

namespace la {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_a;
  const float* lam;
  void* out;
  float* gstate;      // [BH][n_groups][D][D] fp32, transposed (dv-major)
  float* gtot;        // [BH][n_groups] log2 gate total of each group
  double* gprefix;    // [BH][n_groups + 1] exclusive prefix sums of gtot
  void* nodes;        // [BH][n_groups][D][D] element type, transposed
  int64_t T;
  int64_t n_chunks;
  int64_t n_groups;
  int L;
};

constexpr int cilog2(int x) { return x <= 1 ? 0 : 1 + cilog2(x >> 1); }

// Chunk-local inclusive prefix sums of log2(a) for the G chunks of a group,
// into b2s[c*C + i]; zero past the end of the sequence.
template <int C, int G>
__device__ __forceinline__ void gate_prologue(const float* la_bh, int64_t t0, int64_t T, float* b2s) {
  const int w = wave_id(), lane = lane_id();
  for (int c = w; c < G; c += kWaves) {
    const int64_t base = t0 + (int64_t)c * C;
    if constexpr (C <= 64) {
      float x = 0.f;
      if (lane < C && base + lane < T) x = la_bh[base + lane] * kLog2e;
      x = wave_incl_scan(x);
      if (lane < C) b2s[c * C + lane] = x;
    } else {
      static_assert(C == 128, "chunk sizes above 64 must be 128");
      const int64_t i0 = base + 2 * lane;
      const float x0 = i0 < T ? la_bh[i0] * kLog2e : 0.f;
      const float x1 = i0 + 1 < T ? la_bh[i0 + 1] * kLog2e : 0.f;
      const float s = wave_incl_scan(x0 + x1);
      b2s[c * C + 2 * lane] = s - x1;
      b2s[c * C + 2 * lane + 1] = s;
    }
  }
}

// Stage one chunk of K and V into LDS.  Optionally K row-major [C][D] (for
// the score tile), always V^T [D][C] and, when kts != nullptr, K^T [D][C]
// with every key column scaled by exp2(ex_base - b2c[key]) (the gate from the
// key to the point the state is decayed to).  Rows past T are zero.
template <bool BF16, int C, int D>
__device__ __forceinline__ void stage_kv(const typename Elem<BF16>::T* kg, const typename Elem<BF16>::T* vg,
                                         int nv, typename Elem<BF16>::T* Ks, typename Elem<BF16>::T* VT,
                                         typename Elem<BF16>::T* KTs, const float* b2c, float ex_base,
                                         const LdsLayout& lay) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  constexpr int EPV = 16 / sizeof(E);   // elements per 16-byte vector
  constexpr int VPR = D / EPV;          // vectors per row
  for (int idx = threadIdx.x; idx < C * VPR; idx += kWaves * 64) {
    const int r = idx / VPR, cv = idx % VPR;
    uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
    if (r < nv) {
      kx = *reinterpret_cast<const uint4*>(kg + (int64_t)r * D + cv * EPV);
      vx = *reinterpret_cast<const uint4*>(vg + (int64_t)r * D + cv * EPV);
    }
    if (Ks) *reinterpret_cast<uint4*>(Ks + r * lay.ld_row + cv * EPV) = kx;
    const E* ke = reinterpret_cast<const E*>(&kx);
    const E* ve = reinterpret_cast<const E*>(&vx);
    const float u = KTs ? exp2f(ex_base - b2c[r]) : 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      VT[(cv * EPV + e) * lay.ld_t + r] = ve[e];
      if (KTs) KTs[(cv * EPV + e) * lay.ld_t + r] = EL::from_f32(EL::to_f32(ke[e]) * u);
    }
  }
}

// ---------------------------------------------------------------------------
// Group states: A^T[dv][dk] = sum over the group's keys of
// exp2(group_end - key) v k^T, for every group but the last.
template <bool BF16, int C, int D>
__global__ __launch_bounds__(256) void fwd_group_state(FwdArgs a) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  constexpr int G = choose_group(C, D, sizeof(E));
  constexpr int DB = D / 16;
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr LdsLayout lay = lds_layout(C, D, sizeof(E), G, kMaxLevels, false);
  E* VT = reinterpret_cast<E*>(smem + lay.vt);
  E* KTs = reinterpret_cast<E*>(smem + lay.kts);
  float* b2s = reinterpret_cast<float*>(smem + lay.b2);

  const int64_t ng1 = a.n_groups - 1;
  const int64_t bh = blockIdx.x / ng1;
  const int64_t gam = blockIdx.x % ng1;
  const int lane = lane_id(), w = wave_id(), lq = lane >> 4, lr = lane & 15;
  const int64_t T = a.T;
  const int64_t t0 = gam * G * C;
  gate_prologue<C, G>(a.log_a + bh * T, t0, T, b2s);
  __syncthreads();

  float gch[G];
  float gt = 0.f;
#pragma unroll
  for (int c = 0; c < G; ++c) { gch[c] = b2s[c * C + C - 1]; gt += gch[c]; }

  constexpr int MB = (DB + kWaves - 1) / kWaves;   // dv blocks per wave
  f32x4 h[MB][DB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < DB; ++n) h[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const E* kb = reinterpret_cast<const E*>(a.k) + (bh * T + t0) * D;
  const E* vb = reinterpret_cast<const E*>(a.v) + (bh * T + t0) * D;
  float suffix = gt;   // gate from the start of chunk c to the group end
  for (int c = 0; c < G; ++c) {
    suffix -= gch[c];
    __syncthreads();
    // non-last groups are full: every chunk has C valid rows
    stage_kv<BF16, C, D>(kb + (int64_t)c * C * D, vb + (int64_t)c * C * D, C, nullptr, VT, KTs,
                         b2s + c * C, gch[c] + suffix, lay);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int mb = w + m * kWaves;
      if (mb < DB) {
        for (int ks = 0; ks < C; ks += EL::kStep) {
          const auto va = EL::template load_k<C>(VT + (16 * mb + lr) * lay.ld_t + ks + lq * EL::kPerLane, ks + lq * EL::kPerLane);
#pragma unroll
          for (int n = 0; n < DB; ++n) {
            const auto kf = EL::template load_k<C>(KTs + (16 * n + lr) * lay.ld_t + ks + lq * EL::kPerLane, ks + lq * EL::kPerLane);
            h[m][n] = EL::mma(va, kf, h[m][n]);
          }
        }
      }
    }
  }
  float* dst = a.gstate + (bh * a.n_groups + gam) * D * D;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int mb = w + m * kWaves;
    if (mb < DB) {
#pragma unroll
      for (int n = 0; n < DB; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * mb + 4 * lq + i) * D + 16 * n + lr] = h[m][n][i];
    }
  }
  if (threadIdx.x == 0) a.gtot[bh * a.n_groups + gam] = gt;
}

// ---------------------------------------------------------------------------
// Group tree: per (b,h) and state element, walk the groups with the
// binary-counter carry.  node[e] = A_e + sum_{j<=k} decay * bucket_j where
// k = trailing ones of e, i.e. the bucket of 2^k groups ending at e.
constexpr int kMaxTreeLevels = 28;

template <bool BF16>
__global__ __launch_bounds__(256) void fwd_group_tree(FwdArgs a, int D) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  const int DD = D * D;
  const int nblk = (DD + 255) / 256;
  const int64_t bh = blockIdx.x / nblk;
  const int blk = blockIdx.x % nblk;
  const int elem = blk * 256 + threadIdx.x;
  const bool valid = elem < DD;
  const int64_t ng = a.n_groups;
  float slot[kMaxTreeLevels];
  float sc[kMaxTreeLevels];
#pragma unroll
  for (int j = 0; j < kMaxTreeLevels; ++j) { slot[j] = 0.f; sc[j] = 0.f; }
  double pre = 0.0;
  const bool writer = blk == 0 && threadIdx.x == 0;
  const float* gs = a.gstate + bh * ng * DD;
  E* nd = reinterpret_cast<E*>(a.nodes) + bh * ng * DD;
  for (int64_t e = 0; e + 1 < ng; ++e) {
    if (writer) a.gprefix[bh * (ng + 1) + e] = pre;
    const float g = a.gtot[bh * ng + e];
    const float A = valid ? gs[e * DD + elem] : 0.f;
    int kk = 0;
    for (int64_t x = e; x & 1; x >>= 1) ++kk;
    float nw = A;
#pragma unroll
    for (int j = 0; j < kMaxTreeLevels; ++j)
      if (j < kk) nw += exp2f(sc[j] + g) * slot[j];
#pragma unroll
    for (int j = 0; j < kMaxTreeLevels; ++j) {
      if (j == kk) { slot[j] = nw; sc[j] = 0.f; }
      else sc[j] += g;
    }
    if (valid) nd[e * DD + elem] = EL::from_f32(nw);
    pre += (double)g;
  }
  // Consumers read entries 0..ng-1 only (the last group's total is never
  // formed: no later group needs it).
  if (writer) a.gprefix[bh * (ng + 1) + ng - 1] = pre;
}

// ---------------------------------------------------------------------------
// Output kernel: one workgroup per (b,h, group of G chunks).
template <bool BF16, int C, int D>
__global__ __launch_bounds__(256) void fwd_output(FwdArgs a) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  constexpr int G = choose_group(C, D, sizeof(E));
  constexpr int QB = C / 16, DB = D / 16;
  constexpr int LOG2C = cilog2(C), LOG2G = cilog2(G);
  constexpr int NS = LOG2G > 0 ? LOG2G : 1;
  constexpr int KPL = EL::kPerLane;
  extern __shared__ __align__(16) unsigned char smem[];
  const int L = a.L;
  const LdsLayout lay = lds_layout(C, D, sizeof(E), G, L, true);
  E* Qs = reinterpret_cast<E*>(smem + lay.q);
  E* Ks = reinterpret_cast<E*>(smem + lay.k);
  E* VT = reinterpret_cast<E*>(smem + lay.vt);
  E* KTs = G > 1 ? reinterpret_cast<E*>(smem + lay.kts) : nullptr;
  E* SL = G > 1 ? reinterpret_cast<E*>(smem + lay.slots) : nullptr;
  float* lamS = reinterpret_cast<float*>(smem + lay.lam);
  float* b2s = reinterpret_cast<float*>(smem + lay.b2);
  int* gnode = reinterpret_cast<int*>(smem + lay.ginfo);          // [32] node group index or -1
  float* gexp = reinterpret_cast<float*>(smem + lay.ginfo + 128);  // [32] log2 gate to group start

  const int64_t ng = a.n_groups;
  const int64_t bh = blockIdx.x / ng;
  const int64_t gam = blockIdx.x % ng;
  const int lane = lane_id(), w = wave_id(), lq = lane >> 4, lr = lane & 15;
  const int64_t T = a.T;
  const int64_t c0 = gam * G;
  const int nch = (int)(a.n_chunks - c0 < G ? a.n_chunks - c0 : G);
  const int64_t t0 = c0 * C;

  gate_prologue<C, G>(a.log_a + bh * T, t0, T, b2s);
  // Group-level buckets of this group: level LOG2C + LOG2G + i for every set
  // bit i-1 of gam; the node ending at group e_i, gated by the groups between.
  if (threadIdx.x < 32) {
    const int i = threadIdx.x + 1;
    int node = -1;
    float ex = 0.f;
    if (i <= 31 && ((gam >> (i - 1)) & 1)) {
      const int64_t e = ((gam >> i) << i) + (1ll << (i - 1)) - 1;
      node = (int)e;
      const double* gp = a.gprefix + bh * (ng + 1);
      ex = (float)(gp[gam] - gp[e + 1]);
    }
    gnode[threadIdx.x] = node;
    gexp[threadIdx.x] = ex;
  }
  const int nbits = 64 - __builtin_clzll((unsigned long long)gam | 1ull) - (gam == 0 ? 1 : 0);

  const E* qg = reinterpret_cast<const E*>(a.q) + (bh * T + t0) * D;
  const E* kg = reinterpret_cast<const E*>(a.k) + (bh * T + t0) * D;
  const E* vg = reinterpret_cast<const E*>(a.v) + (bh * T + t0) * D;
  E* og = reinterpret_cast<E*>(a.out) + (bh * T + t0) * D;
  const float* lg = a.lam + (bh * T + t0) * L;
  const E* nodes = reinterpret_cast<const E*>(a.nodes) + bh * ng * D * D;

  float sc2[NS];       // log2 lazy gate of chunk-level slot j (level LOG2C + j + 1)
#pragma unroll
  for (int j = 0; j < NS; ++j) sc2[j] = 0.f;
  float pre = 0.f;     // log2 gate from the group start to the current chunk start

  for (int c = 0; c < nch; ++c) {
    const int64_t tc = (int64_t)c * C;   // relative to t0
    const int nv = (int)(T - t0 - tc < C ? T - t0 - tc : C);
    __syncthreads();   // previous chunk's readers are done; prologue visible
    const float* b2c = b2s + c * C;
    const float gch = b2c[C - 1];
    {
      constexpr int EPV = 16 / sizeof(E);
      constexpr int VPR = D / EPV;
      for (int idx = threadIdx.x; idx < C * VPR; idx += kWaves * 64) {
        const int r = idx / VPR, cv = idx % VPR;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (r < nv) x = *reinterpret_cast<const uint4*>(qg + (tc + r) * D + cv * EPV);
        *reinterpret_cast<uint4*>(Qs + r * lay.ld_row + cv * EPV) = x;
      }
      for (int idx = threadIdx.x; idx < C * L; idx += kWaves * 64)
        lamS[idx] = idx < nv * L ? lg[tc * L + idx] : 0.f;
    }
    stage_kv<BF16, C, D>(kg + tc * D, vg + tc * D, nv, Ks, VT, KTs, b2c, gch, lay);
    __syncthreads();

    for (int qb = w; qb < QB; qb += kWaves) {
      f32x4 acc[DB];
#pragma unroll
      for (int n = 0; n < DB; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

      // ---- intra-chunk tile: S^T = K Q^T, masked, kept in registers as P.
      const int iq = 16 * qb + lr;          // this lane's query (column of S^T)
      const float b2q = b2c[iq];
      float P[QB][4];
#pragma unroll
      for (int kb = 0; kb < QB; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) P[kb][i] = 0.f;
        if (kb > qb) continue;
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D; ks += EL::kStep) {
          const auto kf = EL::template load_k<D>(Ks + (16 * kb + lr) * lay.ld_row + ks + lq * KPL, ks + lq * KPL);
          const auto qf = EL::template load_k<D>(Qs + iq * lay.ld_row + ks + lq * KPL, ks + lq * KPL);
          s = EL::mma(kf, qf, s);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 16 * kb + 4 * lq + i;   // key
          if (j <= iq && iq < nv) {
            const int lev = fenwick_level_local((unsigned)iq, (unsigned)j);
            P[kb][i] = s[i] * exp2f(b2q - b2c[j]) * lamS[iq * L + lev];
          }
        }
      }
      // ---- O += P V
      if constexpr (BF16) {
#pragma unroll
        for (int kb = 0; kb < QB; kb += 2) {
          if (kb > qb) continue;
          const bool two = kb + 1 <= qb;
          u16x8 pu;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pu[i] = f32_to_bf16(P[kb][i]);
            pu[4 + i] = two ? f32_to_bf16(P[kb + 1][i]) : (unsigned short)0;
          }
          const bf16x8 pa = __builtin_bit_cast(bf16x8, pu);
#pragma unroll
          for (int n = 0; n < DB; ++n) {
            const E* vrow = VT + (16 * n + lr) * lay.ld_t;
            const u16x4 v0 = *reinterpret_cast<const u16x4*>(vrow + 16 * kb + 4 * lq);
            u16x4 v1 = u16x4{0, 0, 0, 0};
            if (two) v1 = *reinterpret_cast<const u16x4*>(vrow + 16 * (kb + 1) + 4 * lq);
            const u16x8 vu = u16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            acc[n] = EL::mma(pa, __builtin_bit_cast(bf16x8, vu), acc[n]);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < QB; ++kb) {
          if (kb > qb) continue;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int n = 0; n < DB; ++n)
              acc[n] = EL::mma(P[kb][i], VT[(16 * n + lr) * lay.ld_t + 16 * kb + 4 * lq + i], acc[n]);
        }
      }

      // ---- contraction with one bucket state (node^T in [dv][dk] layout)
      auto contract = [&](const E* nodeT, int ldn, int lev, float ex2) {
        f32x4 tmp[DB];
#pragma unroll
        for (int n = 0; n < DB; ++n) tmp[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D; ks += EL::kStep) {
          const auto qf = EL::template load_k<D>(Qs + iq * lay.ld_row + ks + lq * KPL, ks + lq * KPL);
#pragma unroll
          for (int n = 0; n < DB; ++n) {
            const auto nf = EL::template load_k<D>(nodeT + (16 * n + lr) * ldn + ks + lq * KPL, ks + lq * KPL);
            tmp[n] = EL::mma(qf, nf, tmp[n]);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * qb + 4 * lq + i;
          const float wgt = lamS[r * L + lev] * exp2f(b2c[r] + ex2);
#pragma unroll
          for (int n = 0; n < DB; ++n) acc[n][i] += wgt * tmp[n][i];
        }
      };
      // chunk levels inside the group (slots carried in LDS)
      if constexpr (G > 1) {
#pragma unroll
        for (int j = 0; j < NS; ++j)
          if ((c >> j) & 1) contract(SL + j * D * lay.ld_node, lay.ld_node, LOG2C + 1 + j, sc2[j]);
      }
      // group levels (nodes from the tree kernel)
      for (int i = 1; i <= nbits; ++i) {
        const int e = gnode[i - 1];
        if (e >= 0) contract(nodes + (int64_t)e * D * D, D, LOG2C + LOG2G + i, pre + gexp[i - 1]);
      }

      // ---- store the output rows of this query block
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * qb + 4 * lq + i;
        if (r < nv) {
#pragma unroll
          for (int n = 0; n < DB; ++n) og[(tc + r) * D + 16 * n + lr] = EL::from_f32(acc[n][i]);
        }
      }
    }

    // ---- merge this chunk's state into the in-group carry (not after the
    // last chunk of the group: nothing inside the group reads it).
    if constexpr (G > 1) {
      if (c + 1 < nch) {
        int kk = 0;
        for (int x = c; x & 1; x >>= 1) ++kk;     // trailing ones of c
        constexpr int MB = (DB + kWaves - 1) / kWaves;
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const int mb = w + m * kWaves;
          if (mb >= DB) continue;
          f32x4 hh[DB];
#pragma unroll
          for (int n = 0; n < DB; ++n) hh[n] = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int ks = 0; ks < C; ks += EL::kStep) {
            const auto va = EL::template load_k<C>(VT + (16 * mb + lr) * lay.ld_t + ks + lq * KPL, ks + lq * KPL);
#pragma unroll
            for (int n = 0; n < DB; ++n) {
              const auto kf = EL::template load_k<C>(KTs + (16 * n + lr) * lay.ld_t + ks + lq * KPL, ks + lq * KPL);
              hh[n] = EL::mma(va, kf, hh[n]);
            }
          }
          E* dst = SL + kk * D * lay.ld_node;
#pragma unroll
          for (int n = 0; n < DB; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = 16 * mb + 4 * lq + i, col = 16 * n + lr;
              float val = hh[n][i];
#pragma unroll
              for (int j = 0; j < NS; ++j)
                if (j < kk) val += exp2f(sc2[j] + gch) * EL::to_f32(SL[j * D * lay.ld_node + row * lay.ld_node + col]);
              dst[row * lay.ld_node + col] = EL::from_f32(val);
            }
        }
#pragma unroll
        for (int j = 0; j < NS; ++j) sc2[j] = (j == kk) ? 0.f : sc2[j] + gch;
      }
    }
    pre += gch;
  }
}

// ---------------------------------------------------------------------------
// Host-side launch of the three stages for one (dtype, C, D) instantiation.
template <bool BF16, int C, int D>
int launch_fwd_impl(const FwdPlan& p, FwdArgs a, hipStream_t s, hipEvent_t const* ev) {
  using E = typename Elem<BF16>::T;
  constexpr int G = choose_group(C, D, sizeof(E));
  static_assert(G >= 1, "tile does not fit in LDS");
  if (p.G != G) return kEHIP;
  int stage = 0;
  bool ok = true;
  auto mark = [&]() {
    if (ev) ok = ok && hipEventRecord(ev[stage], s) == hipSuccess;
    ++stage;
  };
  if (p.n_groups > 1) {
    const int lds_s = lds_layout(C, D, sizeof(E), G, kMaxLevels, false).total;
    ok = ok && hipFuncSetAttribute((const void*)fwd_group_state<BF16, C, D>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds_s) == hipSuccess;
    if (!ok) return kEHIP;
    mark();
    hipLaunchKernelGGL((fwd_group_state<BF16, C, D>), dim3((unsigned)((p.n_groups - 1) * p.BH)), dim3(256),
                       lds_s, s, a);
    ok = ok && hipGetLastError() == hipSuccess;
    mark();
    hipLaunchKernelGGL((fwd_group_tree<BF16>), dim3((unsigned)(((D * D + 255) / 256) * p.BH)), dim3(256), 0,
                       s, a, D);
    ok = ok && hipGetLastError() == hipSuccess;
  }
  ok = ok && hipFuncSetAttribute((const void*)fwd_output<BF16, C, D>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_out) == hipSuccess;
  if (!ok) return kEHIP;
  mark();
  hipLaunchKernelGGL((fwd_output<BF16, C, D>), dim3((unsigned)(p.n_groups * p.BH)), dim3(256), p.lds_out, s,
                     a);
  ok = ok && hipGetLastError() == hipSuccess;
  if (ev) ok = ok && hipEventRecord(ev[stage], s) == hipSuccess;
  return ok ? kOK : kEHIP;
}

template <bool BF16>
int launch_fwd_dtype(const FwdPlan& p, FwdArgs a, hipStream_t s, hipEvent_t const* ev) {
  constexpr int es = BF16 ? 2 : 4;
  // Shapes whose tiles do not fit in LDS are rejected by plan_fwd and never
  // instantiated here.
#define LA_CASE(CC, DD)                                                        \
  if constexpr (choose_group(CC, DD, es) > 0)                                  \
    if (p.C == CC && p.D == DD) return launch_fwd_impl<BF16, CC, DD>(p, a, s, ev);
  LA_CASE(16, 16) LA_CASE(16, 32) LA_CASE(16, 64) LA_CASE(16, 128)
  LA_CASE(32, 16) LA_CASE(32, 32) LA_CASE(32, 64) LA_CASE(32, 128)
  LA_CASE(64, 16) LA_CASE(64, 32) LA_CASE(64, 64) LA_CASE(64, 128)
  LA_CASE(128, 16) LA_CASE(128, 32) LA_CASE(128, 64) LA_CASE(128, 128)
#undef LA_CASE
  return kESHAPE;
}

}  // namespace la
