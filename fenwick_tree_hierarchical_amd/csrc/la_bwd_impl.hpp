// Backward pass of log-linear Mamba-2 attention for gfx950.
//
// Training needs the gradients of the operator, those of the level weights
// lambda included ("Log-Linear Attention", Spanish summary, section 5
// "Limitaciones", first item).  For a loss with gradient dout with respect to
// O, with A[t,s] = lambda_t^(l(t,s)) M^S[t,s], S = q.k and dP = dout.v:
//   dq_t = sum_s A dP k_s        dk_s = sum_t A dP q_t       dv_s = sum_t A S dout_t
//   dlambda_t^l = sum_{s in bucket l of t} M^S S dP
//   dlog_a_r = sum_{u >= r} (dout_u . o_u - v_u . dv_u),  dout_u . o_u = sum_l lambda_u^l dlambda_u^l.
// The chunking is the forward's (chunks of C tokens, groups of G chunks).
//
// Query side.  The forward's chunk nodes built over (k := v, v := k), i.e.
// N = sum gate * k v^T in (d_k, d_v) order, give dq_t = sum_l lambda gate
// N dout_t and dlambda_t^l = gate q_t . N dout_t, so the forward's state and
// group-tree kernels run unchanged; bwd_chunk_dq forms per chunk the
// intra-chunk tiles and one product per occupied level.
//
// Key side.  The queries that see key s at level l form one aligned block: the
// upper half of the level-l block holding s.  Their weight lambda_t^l belongs
// to the query, so every such block needs a node weighted by its own level:
//   R = sum_{t in block} lambda_t^l gate(block start .. t) q_t dout_t^T.
// Unlike the forward's nodes these do not merge along the tree (the weights
// change with the level).  bwd_rev_states forms the blocks inside a group of G
// chunks, and each group's share of the larger blocks; bwd_rev_tree adds the
// shares up; bwd_chunk_dkv forms the intra-chunk tiles and, per level,
// dk_s += gate(s .. block start) R v_s and dv_s += gate R^T k_s.
// bwd_gate_grad takes the reverse cumulative sum of the per-token gate terms.
//
// Gates are in log2 units as in the forward; every exponent applied is <= 0.
#pragma once

#include "la_bwd_plan.hpp"
#include "la_fwd_impl.hpp"

namespace la {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* log_a;
  const float* lam;
  void* dq;
  void* dk;
  void* dv;
  float* dlog_a;         // [BH][T]: row terms from bwd_chunk_dq, then the gate gradient
  float* dlam;           // [BH][T][L]
  const void* nodes_in;  // query side, forward structure over (v, k): [BH][n_chunks][d_k][d_v]
  const void* nodes;     // [BH][n_groups][d_k][d_v]
  const float* gch;      // [BH][n_chunks] log2 gate total of each chunk
  const double* gprefix; // [BH][n_groups + 1] exclusive prefix sums of the group totals
  void* rnodes_in;       // key side: block starting at chunk x inside a group, [BH][n_chunks][d_k][d_v]
  float* rpart;          // [BH][n_groups][rhalves][JG][d_k][d_v] fp32: a group's share of its group-level blocks
  void* rnodes;          // block starting at group x, [BH][n_groups][d_k][d_v]
  void* rnodes_in_t;     // the same key-side nodes transposed, (d_v, d_k), for the split key-side
  void* rnodes_t;        // kernel; null where the fused kernel runs (it gathers them from R)
  float* dcol;           // [BH][T]: v_s . dv_s
  int64_t T;
  int64_t n_chunks;
  int64_t n_groups;
  int L;
  int JG;                // group levels with an upper block
  int rhalves;           // shares per group and level in rpart: 1, or 2 (one per half group)
};

template <bool BF16, int C, int D>
struct BwdShape {
  using EL = Elem<BF16>;
  static constexpr int NW = bwd_waves(C), NT = 64 * NW;
  static constexpr int QB = C / 16, DB = D / 16;
  static constexpr int NST = QB * (QB + 1) / 2;                // causal 16 x 16 score tiles
  static constexpr int KT = (NST + NW - 1) / NW;               // score tiles per wave (max)
  static constexpr int NCB = DB > NW ? DB / NW : 1;           // output column blocks per wave
  static constexpr int NWA = DB >= NW ? NW : DB;               // waves that own columns
  static constexpr int KSD = (D + EL::kStep - 1) / EL::kStep;   // k-steps over d
  static constexpr int KSC = (C + EL::kStep - 1) / EL::kStep;   // k-steps over tokens
  static constexpr int EPV = 16 / (BF16 ? 2 : 4), VPR = D / EPV, NV = C * VPR;
  static constexpr int NPF = (NV + NT - 1) / NT;
  static constexpr int LOG2C = cilog2(C);
};

// Score tile tau of a chunk -> (later block a, earlier block b), b <= a.
__device__ __forceinline__ void tile_blocks(int tau, int& a, int& b) {
  a = 0;
  while ((a + 1) * (a + 2) / 2 <= tau) ++a;
  b = tau - a * (a + 1) / 2;
}

// Operand fragment of a transposed tile read from a row-major LDS tile: row
// `col` of tile^T (a column of the tile), k-slice of rows k0 .. k0 + KPL - 1;
// zero past `rows`.
template <bool BF16, int ROWS>
__device__ __forceinline__ typename Elem<BF16>::Frag gather_col(const typename Elem<BF16>::T* tile, int ld, int k0,
                                                                int col) {
  if constexpr (BF16) {
    u16x8 f = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (ROWS >= Elem<BF16>::kStep || k0 < ROWS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = tile[(k0 + e) * ld + col];
    }
    return __builtin_bit_cast(bf16x8, f);
  } else {
    return tile[k0 * ld + col];
  }
}

// The same fragment of a transposed D x D node from its row-major copy in
// global memory (row `col` of node^T, k-slice k0 ..): unsigned byte offsets
// from the node's (wave-uniform) base, so the loads take a scalar base.
template <bool BF16, int D>
__device__ __forceinline__ typename Elem<BF16>::Frag gather_node_col(const typename Elem<BF16>::T* node, int k0,
                                                                     int col) {
  using E = typename Elem<BF16>::T;
  const unsigned char* b = reinterpret_cast<const unsigned char*>(node);
  const unsigned o = (unsigned)((k0 * D + col) * (int)sizeof(E));
  if constexpr (BF16) {
    u16x8 f = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (D >= Elem<BF16>::kStep || k0 < D) {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = *reinterpret_cast<const unsigned short*>(b + o + (unsigned)(e * D * 2));
    }
    return __builtin_bit_cast(bf16x8, f);
  } else {
    return *reinterpret_cast<const float*>(b + o);
  }
}

template <bool BF16>
__device__ __forceinline__ typename Elem<BF16>::Frag zero_frag() {
  if constexpr (BF16) return __builtin_bit_cast(bf16x8, u16x8{0, 0, 0, 0, 0, 0, 0, 0});
  else return 0.f;
}

template <bool BF16>
__device__ __forceinline__ void store4(typename Elem<BF16>::T* p, f32x4 x) {
  if constexpr (BF16)
    *reinterpret_cast<u16x4*>(p) = u16x4{f32_to_bf16(x[0]), f32_to_bf16(x[1]), f32_to_bf16(x[2]), f32_to_bf16(x[3])};
  else
    *reinterpret_cast<f32x4*>(p) = x;
}

// Q, K, V and dout rows of chunk `tc` (nv valid rows) into row-major LDS
// tiles, zero past the end; lambda rows into lamS.  NT threads take part.
template <bool BF16, int C, int D, int NT = BwdShape<BF16, C, D>::NT, typename Lay>
__device__ __forceinline__ void bwd_load_chunk(const BwdArgs& a, unsigned char* smem, const Lay& lay,
                                               int64_t bh, int64_t tc, int nv) {
  using SH = BwdShape<BF16, C, D>;
  using E = typename Elem<BF16>::T;
  constexpr int NPF = (SH::NV + NT - 1) / NT;
  const int tid = threadIdx.x;
  const int64_t T = a.T;
  const int L = a.L;
  const void* src[4] = {a.q, a.k, a.v, a.dout};
  const int dst[4] = {lay.q, lay.k, lay.v, lay.g};
  uint4 x[4][NPF];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const E* g = reinterpret_cast<const E*>(src[m]) + (bh * T + tc) * D;
#pragma unroll
    for (int p = 0; p < NPF; ++p) {
      const int idx = tid + p * NT;
      const int r = idx / SH::VPR, cv = idx % SH::VPR;
      x[m][p] = make_uint4(0, 0, 0, 0);
      if (idx < SH::NV && r < nv) x[m][p] = *reinterpret_cast<const uint4*>(g + r * D + cv * SH::EPV);
    }
  }
  const float* lg = a.lam + (bh * T + tc) * L;
  float* lamS = reinterpret_cast<float*>(smem + lay.lam);
  for (int idx = tid; idx < C * L; idx += NT) lamS[idx] = idx < nv * L ? lg[idx] : 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    E* t = reinterpret_cast<E*>(smem + dst[m]);
#pragma unroll
    for (int p = 0; p < NPF; ++p) {
      const int idx = tid + p * NT;
      if (idx < SH::NV) {
        const int r = idx / SH::VPR, cv = idx % SH::VPR;
        *reinterpret_cast<uint4*>(t + r * lay.ld_row + cv * SH::EPV) = x[m][p];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_chunk_dq: one workgroup per (b,h, chunk), laid out like the forward's
// output kernel.  Phase 1 deals the causal 16 x 16 tiles round-robin over the
// waves: dP = dout V^T and S = Q K^T, masked into dS = dP * gate * lambda
// (written over the V tile once every wave is past its V reads) and into the
// lambda gradients of the levels inside the chunk (row sums of S * dP * gate
// per tile).  Phase 2 gives each wave 16 columns of d_k for all rows:
// dq = dS K, then per occupied level Z = dout N^T, dq += lambda * gate * Z
// and the wave's share of the row dot q . Z (the lambda gradient of that
// level).  Shares are added in a fixed order, so results are deterministic.
// Also writes the row terms dout_t . o_t = sum_l lambda_t^l dlambda_t^l.
// bfloat16 tiles up to d = 64 fit four workgroups of four waves per CU in LDS
// and are held to the registers of four waves per SIMD.
template <bool BF16, int C, int D>
constexpr int dq_min_waves() { return BF16 && D <= 64 ? 4 : 1; }

template <bool BF16, int C, int D>
__global__ __launch_bounds__(64 * bwd_waves(C)) __attribute__((amdgpu_waves_per_eu(dq_min_waves<BF16, C, D>(), 8)))
void bwd_chunk_dq(BwdArgs a) {
  using SH = BwdShape<BF16, C, D>;
  using EL = Elem<BF16>;
  using E = typename EL::T;
  using Frag = typename EL::Frag;
  constexpr int QB = SH::QB, DB = SH::DB, KSD = SH::KSD, KSC = SH::KSC, NCB = SH::NCB, NW = SH::NW, KT = SH::KT;
  constexpr int KPL = EL::kPerLane, KST = EL::kStep, LOG2C = SH::LOG2C;
  constexpr int G = state_group(D), LOG2G = cilog2(G);
  constexpr int NPRE = 2;                                      // node fragment buffers
  extern __shared__ __align__(16) unsigned char smem[];
  const int L = a.L;
  const int NI = L - LOG2C - 1;                                // levels above the chunk
  const BwdChunkLds lay = bwd_chunk_lds(C, D, sizeof(E), L, false);
  const E* Qs = reinterpret_cast<const E*>(smem + lay.q);
  const E* Ks = reinterpret_cast<const E*>(smem + lay.k);
  const E* Vs = reinterpret_cast<const E*>(smem + lay.v);
  const E* Gs = reinterpret_cast<const E*>(smem + lay.g);
  E* Ps = reinterpret_cast<E*>(smem + lay.s0);
  const float* lamS = reinterpret_cast<const float*>(smem + lay.lam);
  float* partO = reinterpret_cast<float*>(smem + lay.part);    // [tile][16]: off-diagonal tile row sums
  float* partD = partO + SH::NST * 16;                         // [row block][16][5]: diagonal tile levels 0..4
  float* inter = reinterpret_cast<float*>(smem + lay.inter);   // [wave][level - log2 C - 1][row]
  float* b2c = reinterpret_cast<float*>(smem + lay.b2);

  const int64_t nc = a.n_chunks, ng = a.n_groups, T = a.T;
  const int64_t item = xcd_item(blockIdx.x, gridDim.x);
  const int64_t bh = item / nc, c = item % nc;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id(), lq = lane >> 4, lr = lane & 15;
  const int64_t tc = c * C;
  const int nv = (int)(T - tc < C ? T - tc : C);

  // occupied levels above the chunk, as in the forward: lanes 1..LOG2G hold
  // the chunk levels inside the group, lanes 32..62 the group levels
  const int64_t gam = c / G, cg0 = gam * G;
  const int ci = (int)(c - cg0);
  bool act = false;
  int64_t off = 0;
  int lev = 0, src = 0;
  int64_t eg = 0;
  if (lane >= 1 && lane <= LOG2G) {
    const int j = lane;
    if ((ci >> (j - 1)) & 1) {
      const int el = ((ci >> j) << j) + (1 << (j - 1)) - 1;
      act = true;
      off = (bh * nc + cg0 + el) * D * D;
      src = el + 1;
      lev = LOG2C + j;
    }
  }
  if (lane >= 32 && lane < 63) {
    const int i = lane - 31;
    if (gam > 0 && ((gam >> (i - 1)) & 1)) {
      eg = ((gam >> i) << i) + (1ll << (i - 1)) - 1;
      act = true;
      off = (bh * ng + eg) * D * D;
      lev = LOG2C + LOG2G + i;
    }
  }
  const unsigned long long lmask = __ballot(act);
  const int n_lev = __popcll(lmask);
  const int pos = __popcll(lmask & ((1ull << lane) - 1ull));
  const int ent = __builtin_amdgcn_ds_permute((act ? pos : 63) << 2, lane);
  // occupied levels as a bit mask (every level is below 32)
  unsigned occm = 0;
  for (int li = 0; li < n_lev; ++li)
    occm |= 1u << __builtin_amdgcn_readlane(lev, __builtin_amdgcn_readlane(ent, li));
  const int cb0 = w * NCB;
  const bool owner = cb0 < DB;
  auto node_of = [&](int li) {
    const int el = __builtin_amdgcn_readlane(ent, li);
    const uint64_t o64 = (uint64_t)off;
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)o64, el);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(o64 >> 32), el);
    const int64_t o = (int64_t)(((uint64_t)hi << 32) | lo);
    return (el >= 32 ? reinterpret_cast<const E*>(a.nodes) : reinterpret_cast<const E*>(a.nodes_in)) + o;
  };
  // node fragments as the A operand: row d_k (this wave's columns), k-slice of d_v
  auto load_node = [&](int li, Frag (&dst)[KSD][NCB]) {
    const E* node = node_of(li);
#pragma unroll
    for (int s2 = 0; s2 < KSD; ++s2) {
      const int k0 = s2 * KST + lq * KPL;
#pragma unroll
      for (int n = 0; n < NCB; ++n) dst[s2][n] = EL::template load_k<D>(node + (16 * (cb0 + n) + lr) * D + k0, k0);
    }
  };
  bwd_load_chunk<BF16, C, D>(a, smem, lay, bh, tc, nv);
  if (w == 0) {
    // in-chunk inclusive prefix of log2(a): its exp2 is the gate from the
    // chunk start through each row
    const float x = (lane < C && tc + lane < T) ? a.log_a[bh * T + tc + lane] * kLog2e : 0.f;
    const float y = wave_incl_scan(x);
    if (lane < C) b2c[lane] = y;
  }

  const float gx = (lane < ci) ? a.gch[bh * nc + cg0 + lane] : 0.f;
  const bool grp = act && lane >= 32;
  float g2 = 0.f;
  {
    const float incl = wave_incl_scan(gx);
    float S = __shfl_up(incl, 1, 64);
    if (lane == 0) S = 0.f;
    const float pre = __shfl(S, ci, 64);
    const float Se = __shfl(S, src, 64);
    if (act) {
      if (grp) {
        const double* gp = a.gprefix + bh * (ng + 1);
        g2 = (float)(gp[gam] - gp[eg + 1]) + pre;
      } else {
        g2 = pre - Se;
      }
    }
  }
  __syncthreads();

  // ---- phase 1: transposed score tiles (lane: query row, four keys)
  f32x4 ssv[KT], sdv[KT];
#pragma unroll
  for (int u = 0; u < KT; ++u) {
    ssv[u] = sdv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int tau = w + u * NW;
    if (tau >= SH::NST) break;
    int qb, kb;
    tile_blocks(tau, qb, kb);
    const int iq = 16 * qb + lr;
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      const int k0 = s * KST + lq * KPL;
      const auto kf = EL::template load_k<D>(Ks + (16 * kb + lr) * lay.ld_row + k0, k0);
      const auto qf = EL::template load_k<D>(Qs + iq * lay.ld_row + k0, k0);
      ssv[u] = EL::mma(kf, qf, ssv[u]);
      const auto vf = EL::template load_k<D>(Vs + (16 * kb + lr) * lay.ld_row + k0, k0);
      const auto gf = EL::template load_k<D>(Gs + iq * lay.ld_row + k0, k0);
      sdv[u] = EL::mma(vf, gf, sdv[u]);
    }
  }
  // the Q entries of this wave's columns, for the row dots of the levels
  E qv[QB][NCB][4];
#pragma unroll
  for (int rb = 0; rb < QB; ++rb)
#pragma unroll
    for (int n = 0; n < NCB; ++n) {
      const E* qrow = Qs + (16 * rb + lr) * lay.ld_row + 16 * ((owner ? cb0 : 0) + n) + 4 * lq;
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[rb][n][i] = qrow[i];
    }
  __syncthreads();                                 // Q and V no longer read: row sums and dS go over them
#pragma unroll
  for (int u = 0; u < KT; ++u) {
    const int tau = w + u * NW;
    if (tau >= SH::NST) break;
    int qb, kb;
    tile_blocks(tau, qb, kb);
    const int iq = 16 * qb + lr;
    const int j0 = 16 * kb + 4 * lq;
    const float b2q = b2c[iq];
    float dsv[4], ev[4];
    int lvv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + i;
      int lv = fenwick_level_local((unsigned)iq, (unsigned)j);
      lv = lv < L ? lv : L - 1;
      const float W = __builtin_amdgcn_exp2f(b2q - b2c[j]);
      const bool ok = j <= iq && iq < nv;
      dsv[i] = ok ? sdv[u][i] * W * lamS[iq * L + lv] : 0.f;
      ev[i] = ok ? ssv[u][i] * sdv[u][i] * W : 0.f;
      lvv[i] = lv;
    }
    if constexpr (BF16)
      *reinterpret_cast<u16x4*>(Ps + iq * lay.ld_s + j0) =
          u16x4{f32_to_bf16(dsv[0]), f32_to_bf16(dsv[1]), f32_to_bf16(dsv[2]), f32_to_bf16(dsv[3])};
    else
      *reinterpret_cast<float4*>(Ps + iq * lay.ld_s + j0) = make_float4(dsv[0], dsv[1], dsv[2], dsv[3]);
    if (kb == qb) {
      // inside a 16-block the levels are 0..4
      float dlr[5];
#pragma unroll
      for (int v = 0; v < 5; ++v) {
        dlr[v] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) dlr[v] += (lvv[i] == v) ? ev[i] : 0.f;
        dlr[v] += __shfl_xor(dlr[v], 16, 64);
        dlr[v] += __shfl_xor(dlr[v], 32, 64);
      }
      if (lq == 0) {
#pragma unroll
        for (int v = 0; v < 5; ++v) partD[(qb * 16 + lr) * 5 + v] = dlr[v];
      }
    } else {
      // every key of an earlier 16-block is at one level, 5 + msb(qb ^ kb)
      float es = (ev[0] + ev[1]) + (ev[2] + ev[3]);
      es += __shfl_xor(es, 16, 64);
      es += __shfl_xor(es, 32, 64);
      if (lq == 0) partO[tau * 16 + lr] = es;
    }
  }
  __syncthreads();

  // ---- phase 2: this wave's columns of d_k for all query rows, transposed
  // (lane: query row, four consecutive columns)
  f32x4 acc[QB][NCB];
#pragma unroll
  for (int rb = 0; rb < QB; ++rb)
#pragma unroll
    for (int n = 0; n < NCB; ++n) acc[rb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  Frag nf[NPRE][KSD][NCB];                         // the first levels' node fragments load under dq = dS K
  if (owner) {
#pragma unroll
    for (int u = 0; u < NPRE; ++u)
      if (u < n_lev) load_node(u, nf[u]);
    Frag kt[KSC][NCB];                             // K^T rows (columns of K), k-slices of keys
#pragma unroll
    for (int s = 0; s < KSC; ++s)
#pragma unroll
      for (int n = 0; n < NCB; ++n) kt[s][n] = gather_col<BF16, C>(Ks, lay.ld_row, s * KST + lq * KPL, 16 * (cb0 + n) + lr);
#pragma unroll
    for (int rb = 0; rb < QB; ++rb) {
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        if (s * KST > 16 * rb + 15) break;
        const int k0 = s * KST + lq * KPL;
        Frag pb = zero_frag<BF16>();
        if (k0 < C && k0 / 16 <= rb) pb = EL::load(Ps + (16 * rb + lr) * lay.ld_s + k0);
#pragma unroll
        for (int n = 0; n < NCB; ++n) acc[rb][n] = EL::mma(kt[s][n], pb, acc[rb][n]);
      }
    }
  }
  __syncthreads();                                 // K and dS no longer read: level shares go over them
  if (owner) {
    auto contract = [&](int li, const Frag (&nfr)[KSD][NCB]) {
      const int el = __builtin_amdgcn_readlane(ent, li);
      const float f = __builtin_amdgcn_exp2f(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g2), el)));
      const int lv = __builtin_amdgcn_readlane(lev, el);
#pragma unroll
      for (int rb = 0; rb < QB; ++rb) {
        const int r = 16 * rb + lr;
        f32x4 tmp[NCB];
#pragma unroll
        for (int n = 0; n < NCB; ++n) tmp[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < KSD; ++s2) {
          const int k0 = s2 * KST + lq * KPL;
          const auto gf = EL::template load_k<D>(Gs + r * lay.ld_row + k0, k0);
#pragma unroll
          for (int n = 0; n < NCB; ++n) tmp[n] = EL::mma(nfr[s2][n], gf, tmp[n]);
        }
        const float wq = __builtin_amdgcn_exp2f(b2c[r]) * f;
        const float wl = wq * lamS[r * L + lv];
        float ds = 0.f;
#pragma unroll
        for (int n = 0; n < NCB; ++n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ds += tmp[n][i] * EL::to_f32(qv[rb][n][i]);
            acc[rb][n][i] += wl * tmp[n][i];
          }
        }
        ds += __shfl_xor(ds, 16, 64);
        ds += __shfl_xor(ds, 32, 64);
        if (lq == 0) inter[(w * NI + (lv - LOG2C - 1)) * C + r] = wq * ds;
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int base = 0; base < n_lev; base += NPRE) {
#pragma unroll
      for (int u = 0; u < NPRE; ++u) {
        const int li = base + u;
        if (li >= n_lev) break;
        contract(li, nf[u]);
        if (li + NPRE < n_lev) load_node(li + NPRE, nf[u]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < QB; ++rb) {
      const int r = 16 * rb + lr;
      if (r < nv) {
        E* o = reinterpret_cast<E*>(a.dq) + (bh * T + tc + r) * D + 4 * lq;
#pragma unroll
        for (int n = 0; n < NCB; ++n) store4<BF16>(o + 16 * (cb0 + n), acc[rb][n]);
      }
    }
  }
  __syncthreads();
  // lambda gradients of the chunk's rows: levels 0..4 from the diagonal
  // tiles, 5..log2 C from the earlier tiles of the row block, the rest from
  // the waves' shares; levels with an empty bucket are zero.  Four threads
  // per row, each with a quarter of the levels: they write their entries
  // straight out and add up the row term sum_l lambda_t^l dlambda_t^l with
  // two shuffles.
  static_assert(SH::NT >= 4 * C, "four threads per row");
  {
    const int r = tid >> 2, part = tid & 3;
    const int per = (L + 3) >> 2;
    const int rb = r >> 4, rr = r & 15;
    float rt = 0.f;
    float* dl = a.dlam + (bh * T + tc + r) * L;
    if (r < C) {
      for (int lv = part * per; lv < L && lv < (part + 1) * per; ++lv) {
        float val = 0.f;
        if (lv <= 4 && lv <= LOG2C) {
          val = partD[(rb * 16 + rr) * 5 + lv];
        } else if (lv <= LOG2C) {
          for (int kb = 0; kb < rb; ++kb)
            if (5 + (31 - __builtin_clz((unsigned)(rb ^ kb))) == lv) val += partO[(rb * (rb + 1) / 2 + kb) * 16 + rr];
        } else if ((occm >> lv) & 1u) {
          for (int u = 0; u < SH::NWA; ++u) val += inter[(u * NI + (lv - LOG2C - 1)) * C + r];
        }
        rt += lamS[r * L + lv] * val;
        if (r < nv) dl[lv] = val;
      }
    }
    rt += __shfl_xor(rt, 1, 64);
    rt += __shfl_xor(rt, 2, 64);
    if (r < nv && part == 0) a.dlog_a[bh * T + tc + r] = rt;
  }
}

// ---------------------------------------------------------------------------
// bwd_rev_states: one workgroup per (b,h, group of G chunks).  For every chunk
// level j: the key-side node of each block inside the group that is the upper
// half of its level-j block (chunks whose in-group index has bit j-1 set), and,
// for the group levels whose bit is set in the group index, the group's share
// of its block (gate measured from the group start).  One level at a time, one
// chunk at a time: gated Q^T and dout^T staged transposed, then
// R += dout^T-by-Q products on the matrix cores.
template <bool BF16, int C, int D>
__global__ __launch_bounds__(64 * state_waves(D)) void bwd_rev_states(BwdArgs a) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  constexpr int NW = state_waves(D), NT = 64 * NW, DB = D / 16, HT = DB * DB, TPW = state_tiles_per_wave(D);
  constexpr int G = state_group(D), LOG2G = cilog2(G), LOG2C = cilog2(C);
  constexpr int KPL = EL::kPerLane, KST = EL::kStep, KSC = (C + KST - 1) / KST;
  constexpr int EPV = 16 / (BF16 ? 2 : 4), VPR = D / EPV, NV = C * VPR, NPF = (NV + NT - 1) / NT;
  constexpr RevLds lay = rev_lds(C, D, sizeof(E), G);
  extern __shared__ __align__(16) unsigned char smem[];
  E* QT = reinterpret_cast<E*>(smem + lay.qt);
  E* GT = reinterpret_cast<E*>(smem + lay.gt);
  float* b2s = reinterpret_cast<float*>(smem + lay.b2);

  const int64_t ng = a.n_groups, nc = a.n_chunks, T = a.T;
  const int64_t bh = blockIdx.x / ng, gam = blockIdx.x % ng;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id(), lq = lane >> 4, lr = lane & 15;
  const int L = a.L;
  const int64_t c0 = gam * G;
  const int nch = (int)(nc - c0 < G ? nc - c0 : G);
  const int64_t t0 = c0 * C;
  const float* la_bh = a.log_a + bh * T;
  for (int c = w; c < nch; c += NW) chunk_gate_scan<C>(la_bh, t0 + (int64_t)c * C, T, b2s + c * C);
  __syncthreads();

  const E* qb = reinterpret_cast<const E*>(a.q) + (bh * T + t0) * D;
  const E* gb = reinterpret_cast<const E*>(a.dout) + (bh * T + t0) * D;
  const float* lb = a.lam + (bh * T + t0) * L;
  f32x4 acc[TPW], acct[TPW];       // R and R^T tiles of this wave
  auto zero_acc = [&]() {
#pragma unroll
    for (int h = 0; h < TPW; ++h) acc[h] = acct[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // tiles of R (d_k, d_v) to dst and, when dst_t is given, of R^T (d_v, d_k)
  // to dst_t, both row-major
  auto flush = [&](auto* dst, E* dst_t) {
#pragma unroll
    for (int h = 0; h < TPW; ++h) {
      const int tix = w + h * NW;
      if (tix >= HT) continue;
      const int mb = tix / DB, nb = tix % DB;
      auto* o = dst + (16 * mb + lr) * D + 16 * nb + 4 * lq;
      if constexpr (sizeof(*o) == 4) *reinterpret_cast<f32x4*>(o) = acc[h];
      else store4<BF16>(reinterpret_cast<E*>(o), acc[h]);
      if (dst_t) store4<BF16>(dst_t + (16 * nb + lr) * D + 16 * mb + 4 * lq, acct[h]);
    }
  };
  const int nlev = LOG2G + a.JG;
  const bool keep_t = a.rnodes_in_t != nullptr;   // R^T kept for the split key-side kernel
  for (int j = 1; j <= nlev; ++j) {
    const bool in_group = j <= LOG2G;
    if (!in_group && !((gam >> (j - LOG2G - 1)) & 1)) continue;
    const int lvl = LOG2C + j;
    zero_acc();
    for (int ci = 0; ci < nch; ++ci) {
      if (in_group && !((ci >> (j - 1)) & 1)) continue;
      const int xs = in_group ? ((ci >> (j - 1)) << (j - 1)) : 0;   // block (or group) start
      float pre = 0.f;                                                 // gate from xs to this chunk
      for (int u = xs; u < ci; ++u) pre += b2s[u * C + C - 1];
      const int nvr = (int)(T - t0 - (int64_t)ci * C < C ? T - t0 - (int64_t)ci * C : C);
      // stage Q^T weighted by lambda of the level and the gate, and dout^T
      uint4 qx[NPF], gx[NPF];
      float wr[NPF];
#pragma unroll
      for (int p = 0; p < NPF; ++p) {
        const int idx = tid + p * NT;
        const int r = idx / VPR, cv = idx % VPR;
        qx[p] = gx[p] = make_uint4(0, 0, 0, 0);
        wr[p] = 0.f;
        if (idx < NV && r < nvr) {
          const int64_t off = ((int64_t)ci * C + r) * D + cv * EPV;
          qx[p] = *reinterpret_cast<const uint4*>(qb + off);
          gx[p] = *reinterpret_cast<const uint4*>(gb + off);
          wr[p] = lb[((int64_t)ci * C + r) * L + lvl] * __builtin_amdgcn_exp2f(b2s[ci * C + r] + pre);
        }
      }
#pragma unroll
      for (int p = 0; p < NPF; ++p) {
        const int idx = tid + p * NT;
        if (idx < NV) {
          const int r = idx / VPR, cv = idx % VPR;
          const E* qe = reinterpret_cast<const E*>(&qx[p]);
          const E* ge = reinterpret_cast<const E*>(&gx[p]);
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const int n = cv * EPV + e;
            const int col = r ^ state_swz<C>(n);
            QT[n * lay.ld_t + col] = EL::from_f32(EL::to_f32(qe[e]) * wr[p]);
            GT[n * lay.ld_t + col] = ge[e];
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < TPW; ++h) {
        const int tix = w + h * NW;
        if (tix >= HT) continue;
        const int mb = tix / DB, nb = tix % DB;   // d_k block, d_v block
#pragma unroll
        for (int s = 0; s < KSC; ++s) {
          const int k0 = s * KST + lq * KPL;
          const int ng_ = 16 * nb + lr, nq_ = 16 * mb + lr;
          const auto gf = EL::template load_k<C>(GT + ng_ * lay.ld_t + (k0 ^ state_swz<C>(ng_)), k0);
          const auto qf = EL::template load_k<C>(QT + nq_ * lay.ld_t + (k0 ^ state_swz<C>(nq_)), k0);
          acc[h] = EL::mma(gf, qf, acc[h]);
          if (keep_t) acct[h] = EL::mma(qf, gf, acct[h]);
        }
      }
      __syncthreads();
      const bool last = in_group ? ((((ci + 1) & ((1 << (j - 1)) - 1)) == 0) || ci == nch - 1) : ci == nch - 1;
      if (last) {
        if (in_group) {
          flush(reinterpret_cast<E*>(a.rnodes_in) + (bh * nc + c0 + xs) * D * D,
                keep_t ? reinterpret_cast<E*>(a.rnodes_in_t) + (bh * nc + c0 + xs) * D * D : static_cast<E*>(nullptr));
        } else {
          flush(a.rpart + ((bh * ng + gam) * a.JG + (j - LOG2G - 1)) * D * D, static_cast<E*>(nullptr));
        }
        zero_acc();
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_rev_states_staged: the key-side nodes of bwd_rev_states with every q and
// dout row read from memory once, for bfloat16 shapes whose half groups fit
// twice per CU.  One workgroup per half group (G / 2 chunks).  The half's rows
// are loaded up front (direct global-to-LDS loads into swizzled row-major
// tiles); then, one level at a time, the level's token weights (lambda of the
// level times the gate from the block start) go to LDS and each chunk of the
// level's upper halves adds its products, both operands read as transposed
// fragments (tokens along k) and the weights applied to the Q fragment in
// registers, with the rounding of bwd_rev_states.  Blocks of the in-group
// levels below the top one lie inside a half; the top in-group level's upper
// half is the second half.  For the group levels each half writes its own
// share (gate from the group start) and bwd_rev_tree adds the two.  A wave's
// tiles share their d_k block, so one weighted Q fragment serves all of them.
template <int C, int D>
__global__ __launch_bounds__(64 * state_waves(D)) void bwd_rev_states_staged(BwdArgs a) {
  using EL = Elem<true>;
  using Frag = typename EL::Frag;
  constexpr int NW = state_waves(D), NT = 64 * NW, DB = D / 16, HT = DB * DB, TPW = state_tiles_per_wave(D);
  constexpr int G = state_group(D), GH = G / 2, LOG2G = cilog2(G), LOG2C = cilog2(C);
  constexpr int KST = EL::kStep, KSC = C / KST;
  constexpr int ROWB = 2 * D;                      // bytes per token row
  constexpr RevStagedLds lay = rev_staged_lds(C, D, G);
  static_assert(C % KST == 0 && D >= 64 && GH >= 1 && TPW * NW == HT, "staged rev-states shape");
  static_assert(NW % DB == 0, "a wave's tiles share one d_k block");
  static_assert(GH * C <= NT && G <= NW, "one token row per thread, one gate scan per wave");
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* Qt = smem + lay.q;
  unsigned char* Gt = smem + lay.g;
  float* b2s = reinterpret_cast<float*>(smem + lay.b2);   // gate prefixes of every chunk of the group
  float* wts = reinterpret_cast<float*>(smem + lay.w);    // two buffers of GH * C token weights

  const int64_t ng = a.n_groups, nc = a.n_chunks, T = a.T;
  const int64_t gidx = blockIdx.x >> 1;
  const int half = blockIdx.x & 1;
  const int64_t bh = gidx / ng, gam = gidx % ng;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id(), lq = lane >> 4;
  const int L = a.L, JG = a.JG;
  const int64_t cg0 = gam * G;                                  // the group's first chunk
  const int nchg = (int)(nc - cg0 < G ? nc - cg0 : G);          // chunks in the group
  const int h0 = half * GH;                                     // in-group index of this half's first chunk
  const int nch = nchg - h0 < GH ? nchg - h0 : GH;              // chunks in this half (<= 0: none)
  const int nlev = LOG2G + JG;
  // this half's share of group level j
  auto share = [&](int j) { return a.rpart + (((bh * ng + gam) * 2 + half) * JG + (j - LOG2G - 1)) * D * D; };
  if (nch <= 0) {
    // the group ends inside its first half: this half's shares are zero
    for (int j = LOG2G + 1; j <= nlev; ++j) {
      if (!((gam >> (j - LOG2G - 1)) & 1)) continue;
      f32x4* P = reinterpret_cast<f32x4*>(share(j));
      for (int i = tid; i < D * D / 4; i += NT) P[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int64_t t0 = (cg0 + h0) * C;
  const int nrow = (int)(T - t0 < (int64_t)nch * C ? T - t0 : (int64_t)nch * C);   // rows inside the sequence
  const unsigned char* qsrc = reinterpret_cast<const unsigned char*>(a.q) + (bh * T + t0) * ROWB;
  const unsigned char* gsrc = reinterpret_cast<const unsigned char*>(a.dout) + (bh * T + t0) * ROWB;

  // ---- this half's q and dout rows into LDS
  if (nrow == GH * C) {
    // 1 KB runs: lane l fills granule l mod GPR of row RPR ri + l / GPR with
    // the logical granule that XORs to it (as in the forward's output kernel)
    constexpr int GPR = ROWB / 16, RPR = 1024 / ROWB, RUNS = GH * C * ROWB / 1024;
    static_assert((2 * RUNS) % NW == 0, "runs are dealt evenly over the waves");
    const int lrow = lane / GPR, lg16 = lane % GPR;
    const unsigned off0 = (unsigned)(lrow * ROWB + ((lg16 ^ (lrow & 7)) << 4));
    const unsigned off1 = (unsigned)(lrow * ROWB + ((lg16 ^ ((RPR + lrow) & 7)) << 4));
#pragma unroll
    for (int k = 0; k < 2 * RUNS / NW; ++k) {
      const int run = w + k * NW;                  // wave-uniform
      const int t = run / RUNS, ri = run % RUNS;
      const unsigned o = (RPR >= 8 || (ri & 1) == 0) ? off0 : off1;
      __builtin_amdgcn_global_load_lds((t == 0 ? qsrc : gsrc) + (unsigned)(ri * 1024) + o,
                                       (__attribute__((address_space(3))) void*)((t == 0 ? Qt : Gt) + ri * 1024),
                                       16, 0, 0);
    }
  } else {
    // a half that reaches the end of the sequence: granule copies, zeros past it
    constexpr int GPR = ROWB / 16;
    const int per = nch * C * GPR;
    for (int i = tid; i < 2 * per; i += NT) {
      const int t = i / per, rem = i % per, r = rem / GPR, g = rem % GPR;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (r < nrow) x = *reinterpret_cast<const uint4*>((t == 0 ? qsrc : gsrc) + (size_t)r * ROWB + g * 16);
      *reinterpret_cast<uint4*>((t == 0 ? Qt : Gt) + swz_gran<D>(r, g)) = x;
    }
  }
  // levels with work in this half (wave-uniform): the in-group levels (the
  // top one only in the second half) and the group levels whose bit is set in
  // the group index
  auto next_level = [&](int j) {
    ++j;
    if (j == LOG2G && half == 0) ++j;
    while (j <= nlev && j > LOG2G && !((gam >> (j - LOG2G - 1)) & 1)) ++j;
    return j;
  };
  // one token row per thread; its lambda of the first level is loaded now,
  // that of each next level while the current level's products run
  const int row = tid;
  const bool has_row = row < nrow;
  const float* lrow = a.lam + (bh * T + t0 + row) * L + LOG2C;
  int j = next_level(0);
  float lam_cur = (j <= nlev && has_row) ? lrow[j] : 0.f;

  const float* la_bh = a.log_a + bh * T;
  if (w < nchg) chunk_gate_scan<C>(la_bh, (cg0 + w) * C, T, b2s + w * C);
  __builtin_amdgcn_s_waitcnt(0);                   // this wave's direct loads have landed
  __syncthreads();

  // this wave's tiles: one d_k block mb, d_v blocks nb(h)
  const int mb = w % DB;
  const bool keep_t = a.rnodes_in_t != nullptr;    // R^T kept for the split key-side kernel
  f32x4 acc[TPW], acct[TPW];
#pragma unroll
  for (int h = 0; h < TPW; ++h) acc[h] = acct[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  int buf = 0;
  while (j <= nlev) {
    const bool in_group = j <= LOG2G;
    const int jn = next_level(j);
    float* W = wts + buf * (GH * C);
    buf ^= 1;
    if (row < nch * C) {
      const int cig = h0 + row / C;                // in-group chunk of the row
      float wv = 0.f;
      if (!in_group || ((cig >> (j - 1)) & 1)) {
        const int xs = in_group ? ((cig >> (j - 1)) << (j - 1)) : 0;   // block (or group) start
        float pre = 0.f;                                                 // gate from xs to the chunk
        for (int u = xs; u < cig; ++u) pre += b2s[u * C + C - 1];
        if (has_row) wv = lam_cur * __builtin_amdgcn_exp2f(b2s[h0 * C + row] + pre);
      }
      W[row] = wv;
    }
    __syncthreads();   // W is complete; the other buffer is free once every wave is past this point
    const float lam_nx = (jn <= nlev && has_row) ? lrow[jn] : 0.f;
    for (int ci = 0; ci < nch; ++ci) {
      const int cig = h0 + ci;
      if (in_group && !((cig >> (j - 1)) & 1)) continue;
      const unsigned char* qc = Qt + ci * C * ROWB;
      const unsigned char* gc = Gt + ci * C * ROWB;
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        const float* wr = W + ci * C + s * KST + 8 * lq;   // this lane's eight tokens
        const float4 w0 = *reinterpret_cast<const float4*>(wr);
        const float4 w1 = *reinterpret_cast<const float4*>(wr + 4);
        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        i16x4 lo, hi;
        swz_tr_halves<D>(qc, s * KST, 16 * mb, lane, lo, hi);
        const bf16_t qv[8] = {(bf16_t)lo[0], (bf16_t)lo[1], (bf16_t)lo[2], (bf16_t)lo[3],
                              (bf16_t)hi[0], (bf16_t)hi[1], (bf16_t)hi[2], (bf16_t)hi[3]};
        u16x8 qw;
#pragma unroll
        for (int e = 0; e < 8; ++e) qw[e] = EL::from_f32(EL::to_f32(qv[e]) * wv[e]);
        const Frag qf = __builtin_bit_cast(Frag, qw);
#pragma unroll
        for (int h = 0; h < TPW; ++h) {
          const int nb = (w + h * NW) / DB;
          const Frag gf = swz_tr_frag<D>(gc, s * KST, 16 * nb, lane);
          acc[h] = EL::mma(gf, qf, acc[h]);
          if (in_group && keep_t) acct[h] = EL::mma(qf, gf, acct[h]);   // group shares are stored one way only
        }
      }
      const bool last = in_group ? ((((cig + 1) & ((1 << (j - 1)) - 1)) == 0) || cig == nchg - 1) : ci == nch - 1;
      if (last) {
        const int lr = lane & 15;
        if (in_group) {
          const int xs = (cig >> (j - 1)) << (j - 1);
          bf16_t* R = reinterpret_cast<bf16_t*>(a.rnodes_in) + (bh * nc + cg0 + xs) * D * D;
#pragma unroll
          for (int h = 0; h < TPW; ++h) {
            const int nb = (w + h * NW) / DB;
            store4<true>(R + (16 * mb + lr) * D + 16 * nb + 4 * lq, acc[h]);
            if (keep_t) {
              bf16_t* RT = reinterpret_cast<bf16_t*>(a.rnodes_in_t) + (bh * nc + cg0 + xs) * D * D;
              store4<true>(RT + (16 * nb + lr) * D + 16 * mb + 4 * lq, acct[h]);
            }
          }
        } else {
          float* P = share(j);
#pragma unroll
          for (int h = 0; h < TPW; ++h) {
            const int nb = (w + h * NW) / DB;
            *reinterpret_cast<f32x4*>(P + (16 * mb + lr) * D + 16 * nb + 4 * lq) = acc[h];
          }
        }
#pragma unroll
        for (int h = 0; h < TPW; ++h) acc[h] = acct[h] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    lam_cur = lam_nx;
    j = jn;
  }
}

// ---------------------------------------------------------------------------
// bwd_rev_states_cm: the nodes and shares of bwd_rev_states_staged (d = 64),
// walking the half's chunks once instead of once per level.  A k-step's Q and
// dout fragments are read from LDS once and serve every level the chunk takes
// part in: each in-group level has its own R accumulators (R^T, where it is
// kept, is stored from them), and up to kRevGroupSlots group levels one share
// accumulator each (further group levels take another pass over the chunks).  A pass first writes the token weights
// of all its levels to one table.  Each level adds its products in the order
// of the level-by-level walk, from the same weights, so the results are the
// same bits.
template <int C, int D>
__global__ __launch_bounds__(64 * state_waves(D)) __attribute__((amdgpu_waves_per_eu(4, 8)))
void bwd_rev_states_cm(BwdArgs a) {
  using EL = Elem<true>;
  using Frag = typename EL::Frag;
  constexpr int NW = state_waves(D), NT = 64 * NW, DB = D / 16, HT = DB * DB, TPW = state_tiles_per_wave(D);
  constexpr int G = state_group(D), GH = G / 2, LOG2G = cilog2(G), LOG2C = cilog2(C);
  constexpr int KST = EL::kStep, KSC = C / KST;
  constexpr int ROWB = 2 * D;                      // bytes per token row
  constexpr int GS = kRevGroupSlots, NS = LOG2G + GS;   // weight slots: in-group levels, then group levels
  constexpr int HR = GH * C;                       // token rows of a half
  constexpr int KI = (NS * HR + NT - 1) / NT;      // weight-table entries per thread
  constexpr RevStagedLds lay = rev_cm_lds(C, D, G);
  static_assert(C % KST == 0 && D == 64 && GH >= 1 && TPW * NW == HT, "chunk-major rev-states shape");
  static_assert(NW % DB == 0, "a wave's tiles share one d_k block");
  static_assert(G <= NW, "one gate scan per wave");
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* Qt = smem + lay.q;
  unsigned char* Gt = smem + lay.g;
  float* b2s = reinterpret_cast<float*>(smem + lay.b2);   // gate prefixes of every chunk of the group
  float* wts = reinterpret_cast<float*>(smem + lay.w);    // [NS][HR] token weights of the pass's levels

  const int64_t ng = a.n_groups, nc = a.n_chunks, T = a.T;
  const int64_t gidx = blockIdx.x >> 1;
  const int half = blockIdx.x & 1;
  const int64_t bh = gidx / ng, gam = gidx % ng;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id(), lq = lane >> 4;
  const int L = a.L, JG = a.JG;
  const int64_t cg0 = gam * G;                                  // the group's first chunk
  const int nchg = (int)(nc - cg0 < G ? nc - cg0 : G);          // chunks in the group
  const int h0 = half * GH;                                     // in-group index of this half's first chunk
  const int nch = nchg - h0 < GH ? nchg - h0 : GH;              // chunks in this half (<= 0: none)
  // this half's share of group level j
  auto share = [&](int j) { return a.rpart + (((bh * ng + gam) * 2 + half) * JG + (j - LOG2G - 1)) * D * D; };
  if (nch <= 0) {
    // the group ends inside its first half: this half's shares are zero
    for (int j = LOG2G + 1; j <= LOG2G + JG; ++j) {
      if (!((gam >> (j - LOG2G - 1)) & 1)) continue;
      f32x4* P = reinterpret_cast<f32x4*>(share(j));
      for (int i = tid; i < D * D / 4; i += NT) P[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int64_t t0 = (cg0 + h0) * C;
  const int nrow = (int)(T - t0 < (int64_t)nch * C ? T - t0 : (int64_t)nch * C);   // rows inside the sequence
  const unsigned char* qsrc = reinterpret_cast<const unsigned char*>(a.q) + (bh * T + t0) * ROWB;
  const unsigned char* gsrc = reinterpret_cast<const unsigned char*>(a.dout) + (bh * T + t0) * ROWB;

  // ---- this half's q and dout rows into LDS
  if (nrow == HR) {
    // 1 KB runs: lane l fills granule l mod GPR of row RPR ri + l / GPR with
    // the logical granule that XORs to it
    constexpr int GPR = ROWB / 16, RPR = 1024 / ROWB, RUNS = HR * ROWB / 1024;
    static_assert((2 * RUNS) % NW == 0, "runs are dealt evenly over the waves");
    const int lrow = lane / GPR, lg16 = lane % GPR;
    const unsigned off0 = (unsigned)(lrow * ROWB + ((lg16 ^ (lrow & 7)) << 4));
    const unsigned off1 = (unsigned)(lrow * ROWB + ((lg16 ^ ((RPR + lrow) & 7)) << 4));
#pragma unroll
    for (int k = 0; k < 2 * RUNS / NW; ++k) {
      const int run = w + k * NW;                  // wave-uniform
      const int t = run / RUNS, ri = run % RUNS;
      const unsigned o = (RPR >= 8 || (ri & 1) == 0) ? off0 : off1;
      __builtin_amdgcn_global_load_lds((t == 0 ? qsrc : gsrc) + (unsigned)(ri * 1024) + o,
                                       (__attribute__((address_space(3))) void*)((t == 0 ? Qt : Gt) + ri * 1024),
                                       16, 0, 0);
    }
  } else {
    // a half that reaches the end of the sequence: granule copies, zeros past it
    constexpr int GPR = ROWB / 16;
    const int per = nch * C * GPR;
    for (int i = tid; i < 2 * per; i += NT) {
      const int t = i / per, rem = i % per, r = rem / GPR, g = rem % GPR;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (r < nrow) x = *reinterpret_cast<const uint4*>((t == 0 ? qsrc : gsrc) + (size_t)r * ROWB + g * 16);
      *reinterpret_cast<uint4*>((t == 0 ? Qt : Gt) + swz_gran<D>(r, g)) = x;
    }
  }

  // the group levels with work (the set bits of the group index), GS per pass
  const int ngl = __popcll((unsigned long long)gam);
  const int npass = ngl > GS ? (ngl + GS - 1) / GS : 1;
  unsigned long long gbits = (unsigned long long)gam;          // the set bits not yet walked
  int gl[GS];                                                  // this pass's group levels (0: none)
  auto take_levels = [&]() {
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      gl[g] = gbits ? LOG2G + 1 + __builtin_ctzll(gbits) : 0;
      gbits &= gbits - 1;
    }
  };
  take_levels();
  // level of weight slot sl in this pass (0: no level)
  auto slot_level = [&](int sl, int pass) {
    int j = 0;
#pragma unroll
    for (int g = 0; g < GS; ++g)
      if (sl == LOG2G + g) j = gl[g];
    return sl < LOG2G ? (pass == 0 ? sl + 1 : 0) : j;
  };
  // lambda of each of this thread's table entries, loaded with the rows
  const float* lbase = a.lam + (bh * T + t0) * L + LOG2C;
  float lamv[KI];
  auto load_lambda = [&](int pass) {
#pragma unroll
    for (int k = 0; k < KI; ++k) {
      const int i = tid + k * NT, sl = i / HR, row = i % HR;
      const int j = i < NS * HR ? slot_level(sl, pass) : 0;
      lamv[k] = (j > 0 && row < nrow) ? lbase[(int64_t)row * L + j] : 0.f;
    }
  };
  load_lambda(0);

  const float* la_bh = a.log_a + bh * T;
  if (w < nchg) chunk_gate_scan<C>(la_bh, (cg0 + w) * C, T, b2s + w * C);
  __builtin_amdgcn_s_waitcnt(0);                   // this wave's direct loads have landed
  __syncthreads();

  // this wave's tiles: one d_k block mb, d_v blocks nb(h)
  const int mb = w % DB;
  const bool keep_t = a.rnodes_in_t != nullptr;    // R^T kept for the split key-side kernel
  for (int pass = 0; pass < npass; ++pass) {
    if (pass > 0) {
      __syncthreads();                             // every wave is done with the last pass's table
      take_levels();
      load_lambda(pass);
    }
    // token weights: lambda of the level times the gate from the block (or
    // group) start, zero outside the level's chunks and past the sequence
#pragma unroll
    for (int k = 0; k < KI; ++k) {
      const int i = tid + k * NT, sl = i / HR, row = i % HR;
      if (i >= NS * HR || row >= nch * C) continue;
      const int j = slot_level(sl, pass);
      float wv = 0.f;
      if (j > 0) {
        const bool in_group = j <= LOG2G;
        const int cig = h0 + row / C;
        if (!in_group || ((cig >> (j - 1)) & 1)) {
          const int xs = in_group ? ((cig >> (j - 1)) << (j - 1)) : 0;
          float pre = 0.f;
          for (int u = xs; u < cig; ++u) pre += b2s[u * C + C - 1];
          if (row < nrow) wv = lamv[k] * __builtin_amdgcn_exp2f(b2s[h0 * C + row] + pre);
        }
      }
      wts[i] = wv;
    }
    __syncthreads();

    f32x4 ai[LOG2G][TPW], ag[GS][TPW];
#pragma unroll
    for (int h = 0; h < TPW; ++h) {
#pragma unroll
      for (int l = 0; l < LOG2G; ++l) ai[l][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < GS; ++g) ag[g][h] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int ci = 0; ci < nch; ++ci) {
      const int cig = h0 + ci;
      const unsigned char* qc = Qt + ci * C * ROWB;
      const unsigned char* gc = Gt + ci * C * ROWB;
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        i16x4 lo, hi;
        swz_tr_halves<D>(qc, s * KST, 16 * mb, lane, lo, hi);
        const bf16_t qv[8] = {(bf16_t)lo[0], (bf16_t)lo[1], (bf16_t)lo[2], (bf16_t)lo[3],
                              (bf16_t)hi[0], (bf16_t)hi[1], (bf16_t)hi[2], (bf16_t)hi[3]};
        Frag gf[TPW];
#pragma unroll
        for (int h = 0; h < TPW; ++h) gf[h] = swz_tr_frag<D>(gc, s * KST, 16 * ((w + h * NW) / DB), lane);
        // the Q fragment weighted by slot sl's weights of this lane's eight tokens
        auto weighted = [&](int sl) {
          const float* wr = wts + sl * HR + ci * C + s * KST + 8 * lq;
          const float4 w0 = *reinterpret_cast<const float4*>(wr);
          const float4 w1 = *reinterpret_cast<const float4*>(wr + 4);
          const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
          u16x8 qw;
#pragma unroll
          for (int e = 0; e < 8; ++e) qw[e] = EL::from_f32(EL::to_f32(qv[e]) * wv[e]);
          return __builtin_bit_cast(Frag, qw);
        };
        if (pass == 0) {
#pragma unroll
          for (int l = 0; l < LOG2G; ++l) {
            if (!((cig >> l) & 1)) continue;
            const Frag qf = weighted(l);
#pragma unroll
            for (int h = 0; h < TPW; ++h) ai[l][h] = EL::mma(gf[h], qf, ai[l][h]);
          }
        }
#pragma unroll
        for (int g = 0; g < GS; ++g) {
          if (!gl[g]) continue;
          const Frag qf = weighted(LOG2G + g);
#pragma unroll
          for (int h = 0; h < TPW; ++h) ag[g][h] = EL::mma(gf[h], qf, ag[g][h]);
        }
      }
      const int lr = lane & 15;
      if (pass == 0) {
        // in-group blocks that end with this chunk
#pragma unroll
        for (int l = 0; l < LOG2G; ++l) {
          if (!((cig >> l) & 1)) continue;
          if (!((((cig + 1) & ((1 << l) - 1)) == 0) || cig == nchg - 1)) continue;
          const int xs = (cig >> l) << l;
          bf16_t* R = reinterpret_cast<bf16_t*>(a.rnodes_in) + (bh * nc + cg0 + xs) * D * D;
#pragma unroll
          for (int h = 0; h < TPW; ++h) {
            const int nb = (w + h * NW) / DB;
            store4<true>(R + (16 * mb + lr) * D + 16 * nb + 4 * lq, ai[l][h]);
            // R^T: element i of the lane's four is row 16 nb + 4 lq + i, column 16 mb + lr
            if (keep_t) {
              bf16_t* RT = reinterpret_cast<bf16_t*>(a.rnodes_in_t) + (bh * nc + cg0 + xs) * D * D;
#pragma unroll
              for (int i = 0; i < 4; ++i) RT[(16 * nb + 4 * lq + i) * D + 16 * mb + lr] = f32_to_bf16(ai[l][h][i]);
            }
            ai[l][h] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    }
    // this half's shares of the pass's group levels
    const int lr = lane & 15;
#pragma unroll
    for (int g = 0; g < GS; ++g) {
      if (!gl[g]) continue;
      float* P = share(gl[g]);
#pragma unroll
      for (int h = 0; h < TPW; ++h) {
        const int nb = (w + h * NW) / DB;
        *reinterpret_cast<f32x4*>(P + (16 * mb + lr) * D + 16 * nb + 4 * lq) = ag[g][h];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_rev_tree: the key-side node of every block of groups that is the upper
// half of its level block: it starts at group x >= 1 and spans 2^ctz(x)
// groups; the sum of those groups' shares, each carried by the gate from the
// block start to the group start.  One workgroup per band of 16 rows of one
// node: the band is written as rows of R and, where R^T is kept, through LDS
// (rows padded by one 4-byte word) as 16-element runs of the columns of R^T.
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_rev_tree(BwdArgs a, int D) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  __shared__ E tr[16 * (128 + 4 / sizeof(E))];
  const int ld = D + 4 / (int)sizeof(E);
  const int DD = D * D, nband = D / 16;
  const int64_t ng = a.n_groups;
  const int64_t node = blockIdx.x / nband;
  const int band = blockIdx.x % nband;
  const int64_t bh = node / (ng - 1), x = 1 + node % (ng - 1);
  const int i = __builtin_ctzll((unsigned long long)x);     // block of 2^i groups, group level i + 1
  const int64_t end = x + (1ll << i) < ng ? x + (1ll << i) : ng;
  const double* gp = a.gprefix + bh * (ng + 1);
  const double base = gp[x];
  E* R = reinterpret_cast<E*>(a.rnodes) + (bh * ng + x) * DD;
  const int e0 = band * 16 * D;                             // first element of the band
  const int RH = a.rhalves;
  const size_t hstride = (size_t)a.JG * DD;                 // from a group's first half share to its second
  // four consecutive elements per thread; the shares are loaded four groups
  // at a time, ahead of their weighted adds, which stay in group order
  for (int e4 = threadIdx.x; e4 < 4 * D; e4 += 256) {
    const int e = 4 * e4;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t g0 = x; g0 < end; g0 += 4) {
      f32x4 v[4];
      float wg[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        wg[u] = 0.f;
        if (g0 + u < end) {
          const float* sh = a.rpart + ((bh * ng + g0 + u) * RH * a.JG + i) * DD + e0 + e;
          // the group's share, or the sum of its two halves' shares
          const f32x4 s0 = *reinterpret_cast<const f32x4*>(sh);
          v[u] = RH == 2 ? s0 + *reinterpret_cast<const f32x4*>(sh + hstride) : s0;
          wg[u] = __builtin_amdgcn_exp2f((float)(gp[g0 + u] - base));
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (g0 + u < end) acc += wg[u] * v[u];
    }
    store4<BF16>(R + e0 + e, acc);
#pragma unroll
    for (int k = 0; k < 4; ++k) tr[((e + k) / D) * ld + (e + k) % D] = EL::from_f32(acc[k]);
  }
  if (!a.rnodes_t) return;                                  // workgroup-uniform
  __syncthreads();
  // R^T row j, columns band*16 .. band*16 + 15
  E* RT = reinterpret_cast<E*>(a.rnodes_t) + (bh * ng + x) * DD;
  for (int e = threadIdx.x; e < 16 * D; e += 256) {
    const int j = e / 16, r = e % 16;
    RT[(int64_t)j * D + band * 16 + r] = tr[r * ld + j];
  }
}

// ---------------------------------------------------------------------------
// bwd_chunk_dkv: one workgroup per (b,h, chunk), laid out like bwd_chunk_dq
// with keys in place of queries.  Phase 1 deals the causal tiles over the
// waves (lane: key row, four queries): dS^T = dP * gate * lambda goes to LDS,
// P^T = S * gate * lambda stays in registers.  Phase 2 gives each wave 16
// columns for all key rows: dk = dS^T Q, then P^T is written over dS^T and
// dv = P^T dout; per level above the chunk, dk += gate R v and dv += gate
// R^T k with the key-side node R and its transpose.  Also writes the column
// terms v_s . dv_s (waves' shares added in a fixed order).  Up to d = 64 it
// is held to the registers of three waves per SIMD (the LDS allows three
// workgroups of four waves per CU): measured faster than two waves with a
// deeper node ring; larger tiles would spill.
template <bool BF16, int C, int D>
constexpr int dkv_min_waves() { return D <= 64 ? 3 : 1; }

template <bool BF16, int C, int D>
__global__ __launch_bounds__(64 * bwd_waves(C)) __attribute__((amdgpu_waves_per_eu(dkv_min_waves<BF16, C, D>(), 8)))
void bwd_chunk_dkv(BwdArgs a) {
  using SH = BwdShape<BF16, C, D>;
  using EL = Elem<BF16>;
  using E = typename EL::T;
  using Frag = typename EL::Frag;
  constexpr int QB = SH::QB, DB = SH::DB, KSD = SH::KSD, KSC = SH::KSC, NCB = SH::NCB, NW = SH::NW, KT = SH::KT;
  constexpr int KPL = EL::kPerLane, KST = EL::kStep;
  constexpr int G = state_group(D), LOG2G = cilog2(G);
  constexpr int NPRE = 1;                                      // node fragment buffers
  extern __shared__ __align__(16) unsigned char smem[];
  const int L = a.L;
  const BwdChunkLds lay = bwd_chunk_lds(C, D, sizeof(E), L, true);
  const E* Qs = reinterpret_cast<const E*>(smem + lay.q);
  const E* Ks = reinterpret_cast<const E*>(smem + lay.k);
  const E* Vs = reinterpret_cast<const E*>(smem + lay.v);
  const E* Gs = reinterpret_cast<const E*>(smem + lay.g);
  E* Ss = reinterpret_cast<E*>(smem + lay.s0);                 // dS^T, then P^T
  const float* lamS = reinterpret_cast<const float*>(smem + lay.lam);
  float* colS = reinterpret_cast<float*>(smem + lay.col);      // [wave][key row]
  float* b2c = reinterpret_cast<float*>(smem + lay.b2);
  float* e2c = reinterpret_cast<float*>(smem + lay.e2);

  const int64_t nc = a.n_chunks, ng = a.n_groups, T = a.T;
  const int64_t item = xcd_item(blockIdx.x, gridDim.x);
  const int64_t bh = item / nc, c = item % nc;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id(), lq = lane >> 4, lr = lane & 15;
  const int64_t tc = c * C;
  const int nv = (int)(T - tc < C ? T - tc : C);

  // levels whose upper block lies above the chunk: lanes 1..LOG2G, chunk
  // level j inside the group (bit j-1 of the in-group index clear); lanes
  // 32..62, group level i (bit i-1 of the group index clear)
  const int64_t gam = c / G, cg0 = gam * G;
  const int ci = (int)(c - cg0);
  bool act = false;
  int64_t off = 0;
  int dst_x = 0;
  int64_t xg = 0;
  if (lane >= 1 && lane <= LOG2G) {
    const int j = lane;
    if (!((ci >> (j - 1)) & 1)) {
      const int x = ((ci >> j) << j) + (1 << (j - 1));
      if (cg0 + x < nc) {
        act = true;
        off = (bh * nc + cg0 + x) * D * D;
        dst_x = x;
      }
    }
  }
  if (lane >= 32 && lane < 63) {
    const int i = lane - 31;
    if (!((gam >> (i - 1)) & 1)) {
      xg = ((gam >> i) << i) + (1ll << (i - 1));
      if (xg < ng) {
        act = true;
        off = (bh * ng + xg) * D * D;
      }
    }
  }
  const unsigned long long lmask = __ballot(act);
  const int n_lev = __popcll(lmask);
  const int pos = __popcll(lmask & ((1ull << lane) - 1ull));
  const int ent = __builtin_amdgcn_ds_permute((act ? pos : 63) << 2, lane);
  const int cb0 = w * NCB;
  const bool owner = cb0 < DB;
  // key-side nodes: R rows (d_k) and R^T rows (d_v) of this wave's columns;
  // the first levels' fragments load now, under the tile work
  auto node_off = [&](int li, int& el) {
    el = __builtin_amdgcn_readlane(ent, li);
    const uint64_t o64 = (uint64_t)off;
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)o64, el);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(o64 >> 32), el);
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  auto load_node = [&](int li, Frag (&rf)[KSD][NCB], Frag (&rt)[KSD][NCB]) {
    int el;
    const int64_t o = node_off(li, el);
    const E* R = (el >= 32 ? reinterpret_cast<const E*>(a.rnodes) : reinterpret_cast<const E*>(a.rnodes_in)) + o;
    const E* RT = (el >= 32 ? reinterpret_cast<const E*>(a.rnodes_t) : reinterpret_cast<const E*>(a.rnodes_in_t)) + o;
#pragma unroll
    for (int s2 = 0; s2 < KSD; ++s2) {
      const int k0 = s2 * KST + lq * KPL;
#pragma unroll
      for (int n = 0; n < NCB; ++n) {
        rf[s2][n] = EL::template load_k<D>(R + (16 * (cb0 + n) + lr) * D + k0, k0);
        rt[s2][n] = EL::template load_k<D>(RT + (16 * (cb0 + n) + lr) * D + k0, k0);
      }
    }
  };
  Frag rf[NPRE][KSD][NCB], rt[NPRE][KSD][NCB];
  if (owner) {
#pragma unroll
    for (int u = 0; u < NPRE; ++u)
      if (u < n_lev) load_node(u, rf[u], rt[u]);
  }
  bwd_load_chunk<BF16, C, D>(a, smem, lay, bh, tc, nv);
  if (w == 0) {
    // in-chunk prefix of log2(a), and the gate from each key to the chunk end
    const float x = (lane < C && tc + lane < T) ? a.log_a[bh * T + tc + lane] * kLog2e : 0.f;
    const float y = wave_incl_scan(x);
    const float tot = __shfl(y, C - 1, 64);
    if (lane < C) {
      b2c[lane] = y;
      e2c[lane] = __builtin_amdgcn_exp2f(tot - y);
    }
  }

  float g2 = 0.f;                               // log2 gate from the chunk end to the block start
  if (nc > 1) {
    const float gx = (lane < G && cg0 + lane < nc) ? a.gch[bh * nc + cg0 + lane] : 0.f;
    const float incl = wave_incl_scan(gx);
    float S = __shfl_up(incl, 1, 64);           // S(y): gates of the group's chunks before y
    if (lane == 0) S = 0.f;
    const float after = __shfl(S, ci + 1, 64);
    const float at_x = __shfl(S, dst_x, 64);
    const float at_end = __shfl(S, G, 64);
    if (act) {
      if (lane >= 32) {
        const double* gp = a.gprefix + bh * (ng + 1);
        g2 = (at_end - after) + (float)(gp[xg] - gp[gam + 1]);
      } else {
        g2 = at_x - after;
      }
    }
  }
  __syncthreads();

  // ---- phase 1: tile tau = (query block qb, key block kb <= qb), lane: key
  // row sk, queries t0 .. t0 + 3
  float pT[KT][4];
#pragma unroll
  for (int u = 0; u < KT; ++u) {
#pragma unroll
    for (int i = 0; i < 4; ++i) pT[u][i] = 0.f;
    const int tau = w + u * NW;
    if (tau >= SH::NST) break;
    int qb, kb;
    tile_blocks(tau, qb, kb);
    const int sk = 16 * kb + lr;
    f32x4 ss = f32x4{0.f, 0.f, 0.f, 0.f}, sd = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      const int k0 = s * KST + lq * KPL;
      const auto qf = EL::template load_k<D>(Qs + (16 * qb + lr) * lay.ld_row + k0, k0);
      const auto kf = EL::template load_k<D>(Ks + sk * lay.ld_row + k0, k0);
      ss = EL::mma(qf, kf, ss);
      const auto gf = EL::template load_k<D>(Gs + (16 * qb + lr) * lay.ld_row + k0, k0);
      const auto vf = EL::template load_k<D>(Vs + sk * lay.ld_row + k0, k0);
      sd = EL::mma(gf, vf, sd);
    }
    const int t0 = 16 * qb + 4 * lq;
    const float b2k = b2c[sk];
    float dv_[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + i;
      int lv = fenwick_level_local((unsigned)t, (unsigned)sk);
      lv = lv < L ? lv : L - 1;
      const float W = __builtin_amdgcn_exp2f(b2c[t] - b2k) * lamS[t * L + lv];
      const bool ok = sk <= t && t < nv;
      pT[u][i] = ok ? ss[i] * W : 0.f;
      dv_[i] = ok ? sd[i] * W : 0.f;
    }
    if constexpr (BF16)
      *reinterpret_cast<u16x4*>(Ss + sk * lay.ld_s + t0) =
          u16x4{f32_to_bf16(dv_[0]), f32_to_bf16(dv_[1]), f32_to_bf16(dv_[2]), f32_to_bf16(dv_[3])};
    else
      *reinterpret_cast<float4*>(Ss + sk * lay.ld_s + t0) = make_float4(dv_[0], dv_[1], dv_[2], dv_[3]);
  }
  __syncthreads();

  // ---- phase 2: this wave's columns for all key rows, transposed (lane: key
  // row, four consecutive columns); queries from the key's block on
  f32x4 ak[QB][NCB], av[QB][NCB];
#pragma unroll
  for (int kb = 0; kb < QB; ++kb)
#pragma unroll
    for (int n = 0; n < NCB; ++n) ak[kb][n] = av[kb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // dk = dS^T Q: Q^T rows (columns of Q) as the A operand
  if (owner) {
    Frag ft[KSC][NCB];
#pragma unroll
    for (int s = 0; s < KSC; ++s)
#pragma unroll
      for (int n = 0; n < NCB; ++n) ft[s][n] = gather_col<BF16, C>(Qs, lay.ld_row, s * KST + lq * KPL, 16 * (cb0 + n) + lr);
#pragma unroll
    for (int kb = 0; kb < QB; ++kb) {
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        if (s * KST + KST <= 16 * kb) continue;
        const int k0 = s * KST + lq * KPL;
        Frag sf = zero_frag<BF16>();
        if (k0 < C && k0 / 16 >= kb) sf = EL::load(Ss + (16 * kb + lr) * lay.ld_s + k0);
#pragma unroll
        for (int n = 0; n < NCB; ++n) ak[kb][n] = EL::mma(ft[s][n], sf, ak[kb][n]);
      }
    }
  }
  __syncthreads();                                 // dS^T no longer read: P^T goes over it
#pragma unroll
  for (int u = 0; u < KT; ++u) {
    const int tau = w + u * NW;
    if (tau >= SH::NST) break;
    int qb, kb;
    tile_blocks(tau, qb, kb);
    const int sk = 16 * kb + lr, t0 = 16 * qb + 4 * lq;
    if constexpr (BF16)
      *reinterpret_cast<u16x4*>(Ss + sk * lay.ld_s + t0) =
          u16x4{f32_to_bf16(pT[u][0]), f32_to_bf16(pT[u][1]), f32_to_bf16(pT[u][2]), f32_to_bf16(pT[u][3])};
    else
      *reinterpret_cast<float4*>(Ss + sk * lay.ld_s + t0) = make_float4(pT[u][0], pT[u][1], pT[u][2], pT[u][3]);
  }
  __syncthreads();
  if (owner) {
    // dv = P^T dout: dout^T rows as the A operand
    Frag ft[KSC][NCB];
#pragma unroll
    for (int s = 0; s < KSC; ++s)
#pragma unroll
      for (int n = 0; n < NCB; ++n) ft[s][n] = gather_col<BF16, C>(Gs, lay.ld_row, s * KST + lq * KPL, 16 * (cb0 + n) + lr);
#pragma unroll
    for (int kb = 0; kb < QB; ++kb) {
#pragma unroll
      for (int s = 0; s < KSC; ++s) {
        if (s * KST + KST <= 16 * kb) continue;
        const int k0 = s * KST + lq * KPL;
        Frag sf = zero_frag<BF16>();
        if (k0 < C && k0 / 16 >= kb) sf = EL::load(Ss + (16 * kb + lr) * lay.ld_s + k0);
#pragma unroll
        for (int n = 0; n < NCB; ++n) av[kb][n] = EL::mma(ft[s][n], sf, av[kb][n]);
      }
    }
    auto contract = [&](int li, const Frag (&rf)[KSD][NCB], const Frag (&rt)[KSD][NCB]) {
      const int el = __builtin_amdgcn_readlane(ent, li);
      const float f = __builtin_amdgcn_exp2f(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g2), el)));
#pragma unroll
      for (int kb = 0; kb < QB; ++kb) {
        const int sk = 16 * kb + lr;
        f32x4 tk[NCB], tv[NCB];
#pragma unroll
        for (int n = 0; n < NCB; ++n) tk[n] = tv[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < KSD; ++s2) {
          const int k0 = s2 * KST + lq * KPL;
          const auto vf = EL::template load_k<D>(Vs + sk * lay.ld_row + k0, k0);
          const auto kf = EL::template load_k<D>(Ks + sk * lay.ld_row + k0, k0);
#pragma unroll
          for (int n = 0; n < NCB; ++n) {
            tk[n] = EL::mma(rf[s2][n], vf, tk[n]);
            tv[n] = EL::mma(rt[s2][n], kf, tv[n]);
          }
        }
        const float wk = f * e2c[sk];
#pragma unroll
        for (int n = 0; n < NCB; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ak[kb][n][i] += wk * tk[n][i];
            av[kb][n][i] += wk * tv[n][i];
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int base = 0; base < n_lev; base += NPRE) {
#pragma unroll
      for (int u = 0; u < NPRE; ++u) {
        const int li = base + u;
        if (li >= n_lev) break;
        contract(li, rf[u], rt[u]);
        if (li + NPRE < n_lev) load_node(li + NPRE, rf[u], rt[u]);
      }
    }
    // this wave's share of v_s . dv_s, then the rows of dk and dv
#pragma unroll
    for (int kb = 0; kb < QB; ++kb) {
      const int sk = 16 * kb + lr;
      float cs = 0.f;
#pragma unroll
      for (int n = 0; n < NCB; ++n) {
        const E* vrow = Vs + sk * lay.ld_row + 16 * (cb0 + n) + 4 * lq;
#pragma unroll
        for (int i = 0; i < 4; ++i) cs += av[kb][n][i] * EL::to_f32(vrow[i]);
      }
      cs += __shfl_xor(cs, 16, 64);
      cs += __shfl_xor(cs, 32, 64);
      if (lq == 0) colS[w * C + sk] = cs;
      if (sk < nv) {
        E* ok = reinterpret_cast<E*>(a.dk) + (bh * T + tc + sk) * D + 4 * lq;
        E* ov = reinterpret_cast<E*>(a.dv) + (bh * T + tc + sk) * D + 4 * lq;
#pragma unroll
        for (int n = 0; n < NCB; ++n) {
          store4<BF16>(ok + 16 * (cb0 + n), ak[kb][n]);
          store4<BF16>(ov + 16 * (cb0 + n), av[kb][n]);
        }
      }
    }
  }
  __syncthreads();
  if (tid < nv) {
    float cs = 0.f;
    for (int u = 0; u < SH::NWA; ++u) cs += colS[u * C + tid];
    a.dcol[bh * T + tc + tid] = cs;
  }
}

// ---------------------------------------------------------------------------
// bwd_chunk_fused: bwd_chunk_dq and bwd_chunk_dkv in one workgroup of twice
// their waves, for the bf16 shapes where two such workgroups fit per CU.  The
// chunk is loaded once and its causal score tiles are formed once, in both
// orientations: dS by query row (for dq), dS^T and P^T by key row (for dk and
// dv), and the in-chunk shares of the lambda gradients.  Then the first half
// of the waves runs the query side (dq = dS K and the levels of the forward
// structure over (v, k)) while the second half runs the key side (dk = dS^T Q,
// dv = P^T dout and the key-side nodes).  Each side's arithmetic is that of
// its own kernel, so the results are the same bits; the key-side nodes must
// be complete when it starts.
// Tile reads of the fused kernel.  DIR: the chunk's tiles arrived by direct
// global-to-LDS loads into swizzled rows of 2 D bytes (granule g of row r at
// g ^ (r mod 8)); else they are padded rows of ld_row elements.
template <bool BF16, int D, bool DIR>
__device__ __forceinline__ typename Elem<BF16>::Frag fused_row(const unsigned char* tile, int ld_row, int r, int k0) {
  using EL = Elem<BF16>;
  if constexpr (DIR) return __builtin_bit_cast(typename EL::Frag, *reinterpret_cast<const u16x8*>(tile + swz_gran<D>(r, k0 / 8)));
  else return EL::template load_k<D>(reinterpret_cast<const typename EL::T*>(tile) + r * ld_row + k0, k0);
}
// Column c0 + (lane mod 16) of the tile as an operand fragment over rows
// kb + 8 (lane / 16) .. + 7 (ROWS rows in the tile).
template <bool BF16, int ROWS, int D, bool DIR>
__device__ __forceinline__ typename Elem<BF16>::Frag fused_col(const unsigned char* tile, int ld_row, int kb, int c0,
                                                               int lane) {
  using EL = Elem<BF16>;
  if constexpr (DIR) return swz_tr_frag<D>(tile, kb, c0, lane);
  else return gather_col<BF16, ROWS>(reinterpret_cast<const typename EL::T*>(tile), ld_row, kb + (lane >> 4) * EL::kPerLane,
                                     c0 + (lane & 15));
}
// The four consecutive entries of row r from column c (c a multiple of 4).
template <bool BF16, int D, bool DIR>
__device__ __forceinline__ const typename Elem<BF16>::T* fused_quad(const unsigned char* tile, int ld_row, int r, int c) {
  using T = typename Elem<BF16>::T;
  if constexpr (DIR) return reinterpret_cast<const T*>(tile + swz_gran<D>(r, c / 8) + (c % 8) * (int)sizeof(T));
  else return reinterpret_cast<const T*>(tile) + r * ld_row + c;
}

//
// NT: the query-side nodes are the forward's own (saved by the caller's
// forward pass over (k, v)), which hold the transposes of the nodes over
// (v, k): their fragments are gathered from the columns, as the key side's
// R^T fragments are.
template <bool BF16, int C, int D, bool NT = false>
__global__ __launch_bounds__(128 * bwd_waves(C)) void bwd_chunk_fused(BwdArgs a) {
  using SH = BwdShape<BF16, C, D>;
  using EL = Elem<BF16>;
  using E = typename EL::T;
  using Frag = typename EL::Frag;
  constexpr int QB = SH::QB, DB = SH::DB, KSD = SH::KSD, KSC = SH::KSC, NCB = SH::NCB, NW = SH::NW;
  constexpr int KPL = EL::kPerLane, KST = EL::kStep, LOG2C = SH::LOG2C;
  constexpr int NW2 = 2 * NW, NT2 = 64 * NW2;
  constexpr int KT2 = (SH::NST + NW2 - 1) / NW2;              // score tiles per wave (max)
  constexpr int G = state_group(D), LOG2G = cilog2(G);
  static_assert(64 * NW >= 4 * C, "four query-side threads per row");
  extern __shared__ __align__(16) unsigned char smem[];
  const int L = a.L;
  const int NI = L - LOG2C - 1;                                // levels above the chunk
  const BwdFusedLds lay = bwd_fused_lds(C, D, sizeof(E), L);
  // d = 64: the chunk's tiles arrive by direct global-to-LDS loads into
  // swizzled rows (inside the padded regions of the plan)
  constexpr bool DIR = BF16 && D == 64 && C >= 32;
  const unsigned char* Qt = smem + lay.q;
  const unsigned char* Kt = smem + lay.k;
  const unsigned char* Vt = smem + lay.v;
  const unsigned char* Gt = smem + lay.g;
  E* S0 = reinterpret_cast<E*>(smem + lay.s0);                 // dS by query row
  E* S1 = reinterpret_cast<E*>(smem + lay.s1);                 // dS^T by key row
  E* S2 = reinterpret_cast<E*>(smem + lay.s2);                 // P^T by key row
  const float* lamS = reinterpret_cast<const float*>(smem + lay.lam);
  float* partO = reinterpret_cast<float*>(smem + lay.part);    // [tile][16]: off-diagonal tile row sums
  float* partD = partO + SH::NST * 16;                         // [row block][16][5]: diagonal tile levels 0..4
  float* inter = reinterpret_cast<float*>(smem + lay.inter);   // [wave][level - log2 C - 1][row]
  float* colS = reinterpret_cast<float*>(smem + lay.col);      // [wave][key row]
  float* b2c = reinterpret_cast<float*>(smem + lay.b2);
  float* e2c = reinterpret_cast<float*>(smem + lay.e2);

  const int64_t nc = a.n_chunks, ng = a.n_groups, T = a.T;
  const int64_t item = xcd_item(blockIdx.x, gridDim.x);
  const int64_t bh = item / nc, c = item % nc;
  const int tid = threadIdx.x, lane = lane_id(), wg = wave_id(), lq = lane >> 4, lr = lane & 15;
  const bool qside = wg < NW;                                  // wave-uniform
  const int w = qside ? wg : wg - NW;                          // wave index within its side
  const int64_t tc = c * C;
  const int nv = (int)(T - tc < C ? T - tc : C);
  const int64_t gam = c / G, cg0 = gam * G;
  const int ci = (int)(c - cg0);

  if constexpr (DIR) {
    constexpr int ROWB = 2 * D, GPR = ROWB / 16, RPR = 1024 / ROWB, RUNS = C * ROWB / 1024;
    static_assert(RPR == 8 && (4 * RUNS) % NW2 == 0, "1 KB runs of eight rows, dealt evenly over the waves");
    const unsigned char* src[4] = {static_cast<const unsigned char*>(a.q), static_cast<const unsigned char*>(a.k),
                                   static_cast<const unsigned char*>(a.v), static_cast<const unsigned char*>(a.dout)};
    const int dst[4] = {lay.q, lay.k, lay.v, lay.g};
    const size_t cbase = (size_t)(bh * T + tc) * ROWB;
    if (nv == C) {
      // lane l fills granule l mod GPR of row l / GPR of each run with the
      // logical granule that XORs to it (the same offset in every run)
      const int lrow = lane / GPR, lg16 = lane % GPR;
      const unsigned off = (unsigned)(lrow * ROWB + ((lg16 ^ (lrow & 7)) << 4));
#pragma unroll
      for (int k = 0; k < 4 * RUNS / NW2; ++k) {
        const int run = wg + k * NW2;              // wave-uniform
        const int t = run / RUNS, ri = run % RUNS;
        __builtin_amdgcn_global_load_lds(src[t] + cbase + (unsigned)(ri * 1024) + off,
                                         (__attribute__((address_space(3))) void*)(smem + dst[t] + ri * 1024), 16, 0, 0);
      }
    } else {
      // the partial last chunk: granule copies, zeros past the sequence
      for (int i = tid; i < 4 * C * GPR; i += NT2) {
        const int t = i / (C * GPR), rem = i % (C * GPR), r = rem / GPR, g = rem % GPR;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (r < nv) x = *reinterpret_cast<const uint4*>(src[t] + cbase + (size_t)r * ROWB + g * 16);
        *reinterpret_cast<uint4*>(smem + dst[t] + swz_gran<D>(r, g)) = x;
      }
    }
    const float* lg = a.lam + (bh * T + tc) * L;
    float* lamW = reinterpret_cast<float*>(smem + lay.lam);
    for (int idx = tid; idx < C * L; idx += NT2) lamW[idx] = idx < nv * L ? lg[idx] : 0.f;
  } else {
    bwd_load_chunk<BF16, C, D, NT2>(a, smem, lay, bh, tc, nv);
  }
  if (wg == 0) {
    // in-chunk inclusive prefix of log2(a), and the gate from each key to the
    // chunk end
    const float x = (lane < C && tc + lane < T) ? a.log_a[bh * T + tc + lane] * kLog2e : 0.f;
    const float y = wave_incl_scan(x);
    const float tot = __shfl(y, C - 1, 64);
    if (lane < C) {
      b2c[lane] = y;
      e2c[lane] = __builtin_amdgcn_exp2f(tot - y);
    }
  }
  if constexpr (DIR) __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads have landed
  __syncthreads();

  // ---- phase 1: tile tau = (query block qb, key block kb <= qb), S and dP
  // with a lane per query (four keys) and with a lane per key (four queries)
#pragma unroll
  for (int u = 0; u < KT2; ++u) {
    const int tau = wg + u * NW2;
    if (tau >= SH::NST) break;
    int qb, kb;
    tile_blocks(tau, qb, kb);
    f32x4 sq = f32x4{0.f, 0.f, 0.f, 0.f}, dpq = sq, sk = sq, dpk = sq;
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      const int k0 = s * KST + lq * KPL;
      const auto kf = fused_row<BF16, D, DIR>(Kt, lay.ld_row, 16 * kb + lr, k0);
      const auto qf = fused_row<BF16, D, DIR>(Qt, lay.ld_row, 16 * qb + lr, k0);
      const auto vf = fused_row<BF16, D, DIR>(Vt, lay.ld_row, 16 * kb + lr, k0);
      const auto gf = fused_row<BF16, D, DIR>(Gt, lay.ld_row, 16 * qb + lr, k0);
      sq = EL::mma(kf, qf, sq);
      dpq = EL::mma(vf, gf, dpq);
      sk = EL::mma(qf, kf, sk);
      dpk = EL::mma(gf, vf, dpk);
    }
    {
      // query side: dS rows and the in-chunk lambda gradient shares
      const int iq = 16 * qb + lr;
      const int j0 = 16 * kb + 4 * lq;
      const float b2q = b2c[iq];
      float dsv[4], ev[4];
      int lvv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + i;
        int lv = fenwick_level_local((unsigned)iq, (unsigned)j);
        lv = lv < L ? lv : L - 1;
        const float W = __builtin_amdgcn_exp2f(b2q - b2c[j]);
        const bool ok = j <= iq && iq < nv;
        dsv[i] = ok ? dpq[i] * W * lamS[iq * L + lv] : 0.f;
        ev[i] = ok ? sq[i] * dpq[i] * W : 0.f;
        lvv[i] = lv;
      }
      *reinterpret_cast<u16x4*>(S0 + iq * lay.ld_s + j0) =
          u16x4{f32_to_bf16(dsv[0]), f32_to_bf16(dsv[1]), f32_to_bf16(dsv[2]), f32_to_bf16(dsv[3])};
      if (kb == qb) {
        // inside a 16-block the levels are 0..4
        float dlr[5];
#pragma unroll
        for (int v = 0; v < 5; ++v) {
          dlr[v] = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) dlr[v] += (lvv[i] == v) ? ev[i] : 0.f;
          dlr[v] += __shfl_xor(dlr[v], 16, 64);
          dlr[v] += __shfl_xor(dlr[v], 32, 64);
        }
        if (lq == 0) {
#pragma unroll
          for (int v = 0; v < 5; ++v) partD[(qb * 16 + lr) * 5 + v] = dlr[v];
        }
      } else {
        // every key of an earlier 16-block is at one level, 5 + msb(qb ^ kb)
        float es = (ev[0] + ev[1]) + (ev[2] + ev[3]);
        es += __shfl_xor(es, 16, 64);
        es += __shfl_xor(es, 32, 64);
        if (lq == 0) partO[tau * 16 + lr] = es;
      }
    }
    {
      // key side: dS^T and P^T rows
      const int skr = 16 * kb + lr, t0 = 16 * qb + 4 * lq;
      const float b2k = b2c[skr];
      float pv[4], dv_[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + i;
        int lv = fenwick_level_local((unsigned)t, (unsigned)skr);
        lv = lv < L ? lv : L - 1;
        const float W = __builtin_amdgcn_exp2f(b2c[t] - b2k) * lamS[t * L + lv];
        const bool ok = skr <= t && t < nv;
        pv[i] = ok ? sk[i] * W : 0.f;
        dv_[i] = ok ? dpk[i] * W : 0.f;
      }
      *reinterpret_cast<u16x4*>(S1 + skr * lay.ld_s + t0) =
          u16x4{f32_to_bf16(dv_[0]), f32_to_bf16(dv_[1]), f32_to_bf16(dv_[2]), f32_to_bf16(dv_[3])};
      *reinterpret_cast<u16x4*>(S2 + skr * lay.ld_s + t0) =
          u16x4{f32_to_bf16(pv[0]), f32_to_bf16(pv[1]), f32_to_bf16(pv[2]), f32_to_bf16(pv[3])};
    }
  }
  __syncthreads();

  const int cb0 = w * NCB;
  const bool owner = cb0 < DB;
  unsigned occm = 0;                               // query side: occupied levels as a bit mask
  if (qside) {
    // ---- query side: occupied levels above the chunk, as in the forward
    bool act = false;
    int64_t off = 0;
    int lev = 0, src = 0;
    int64_t eg = 0;
    if (lane >= 1 && lane <= LOG2G) {
      const int j = lane;
      if ((ci >> (j - 1)) & 1) {
        const int el = ((ci >> j) << j) + (1 << (j - 1)) - 1;
        act = true;
        off = (bh * nc + cg0 + el) * D * D;
        src = el + 1;
        lev = LOG2C + j;
      }
    }
    if (lane >= 32 && lane < 63) {
      const int i = lane - 31;
      if (gam > 0 && ((gam >> (i - 1)) & 1)) {
        eg = ((gam >> i) << i) + (1ll << (i - 1)) - 1;
        act = true;
        off = (bh * ng + eg) * D * D;
        lev = LOG2C + LOG2G + i;
      }
    }
    const unsigned long long lmask = __ballot(act);
    const int n_lev = __popcll(lmask);
    const int pos = __popcll(lmask & ((1ull << lane) - 1ull));
    const int ent = __builtin_amdgcn_ds_permute((act ? pos : 63) << 2, lane);
    for (int li = 0; li < n_lev; ++li)
      occm |= 1u << __builtin_amdgcn_readlane(lev, __builtin_amdgcn_readlane(ent, li));
    auto node_of = [&](int li) {
      const int el = __builtin_amdgcn_readlane(ent, li);
      const uint64_t o64 = (uint64_t)off;
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)o64, el);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(o64 >> 32), el);
      const int64_t o = (int64_t)(((uint64_t)hi << 32) | lo);
      return (el >= 32 ? reinterpret_cast<const E*>(a.nodes) : reinterpret_cast<const E*>(a.nodes_in)) + o;
    };
    constexpr int NPRE = 2;
    auto load_node = [&](int li, Frag (&dst)[KSD][NCB]) {
      const E* node = node_of(li);
#pragma unroll
      for (int s2 = 0; s2 < KSD; ++s2) {
        const int k0 = s2 * KST + lq * KPL;
#pragma unroll
        for (int n = 0; n < NCB; ++n) {
          if constexpr (NT) dst[s2][n] = gather_node_col<BF16, D>(node, k0, 16 * (cb0 + n) + lr);
          else dst[s2][n] = EL::template load_k<D>(node + (16 * (cb0 + n) + lr) * D + k0, k0);
        }
      }
    };
    const float gx = (lane < ci) ? a.gch[bh * nc + cg0 + lane] : 0.f;
    const bool grp = act && lane >= 32;
    float g2 = 0.f;
    {
      const float incl = wave_incl_scan(gx);
      float S = __shfl_up(incl, 1, 64);
      if (lane == 0) S = 0.f;
      const float pre = __shfl(S, ci, 64);
      const float Se = __shfl(S, src, 64);
      if (act) {
        if (grp) {
          const double* gp = a.gprefix + bh * (ng + 1);
          g2 = (float)(gp[gam] - gp[eg + 1]) + pre;
        } else {
          g2 = pre - Se;
        }
      }
    }
    if (owner) {
      Frag nf[NPRE][KSD][NCB];
      // row loads: a ring of NPRE nodes ahead; gathers (the forward's nodes)
      // take twice the registers in flight, so one node ahead
#pragma unroll
      for (int u = 0; u < (NT ? 1 : NPRE); ++u)
        if (u < n_lev) load_node(u, nf[u]);
      f32x4 acc[QB][NCB];
#pragma unroll
      for (int rb = 0; rb < QB; ++rb)
#pragma unroll
        for (int n = 0; n < NCB; ++n) acc[rb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        Frag kt[KSC][NCB];                         // K^T rows (columns of K), k-slices of keys
#pragma unroll
        for (int s = 0; s < KSC; ++s)
#pragma unroll
          for (int n = 0; n < NCB; ++n)
            kt[s][n] = fused_col<BF16, C, D, DIR>(Kt, lay.ld_row, s * KST, 16 * (cb0 + n), lane);
#pragma unroll
        for (int rb = 0; rb < QB; ++rb) {
#pragma unroll
          for (int s = 0; s < KSC; ++s) {
            if (s * KST > 16 * rb + 15) break;
            const int k0 = s * KST + lq * KPL;
            Frag pb = zero_frag<BF16>();
            if (k0 < C && k0 / 16 <= rb) pb = EL::load(S0 + (16 * rb + lr) * lay.ld_s + k0);
#pragma unroll
            for (int n = 0; n < NCB; ++n) acc[rb][n] = EL::mma(kt[s][n], pb, acc[rb][n]);
          }
        }
      }
      // the Q entries of this wave's columns, for the row dots of the levels
      E qv[QB][NCB][4];
#pragma unroll
      for (int rb = 0; rb < QB; ++rb)
#pragma unroll
        for (int n = 0; n < NCB; ++n) {
          const E* qrow = fused_quad<BF16, D, DIR>(Qt, lay.ld_row, 16 * rb + lr, 16 * (cb0 + n) + 4 * lq);
#pragma unroll
          for (int i = 0; i < 4; ++i) qv[rb][n][i] = qrow[i];
        }
      auto contract = [&](int li, const Frag (&nfr)[KSD][NCB]) {
        const int el = __builtin_amdgcn_readlane(ent, li);
        const float f = __builtin_amdgcn_exp2f(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g2), el)));
        const int lv = __builtin_amdgcn_readlane(lev, el);
#pragma unroll
        for (int rb = 0; rb < QB; ++rb) {
          const int r = 16 * rb + lr;
          f32x4 tmp[NCB];
#pragma unroll
          for (int n = 0; n < NCB; ++n) tmp[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s2 = 0; s2 < KSD; ++s2) {
            const int k0 = s2 * KST + lq * KPL;
            const auto gf = fused_row<BF16, D, DIR>(Gt, lay.ld_row, r, k0);
#pragma unroll
            for (int n = 0; n < NCB; ++n) tmp[n] = EL::mma(nfr[s2][n], gf, tmp[n]);
          }
          const float wq = __builtin_amdgcn_exp2f(b2c[r]) * f;
          const float wl = wq * lamS[r * L + lv];
          float ds = 0.f;
#pragma unroll
          for (int n = 0; n < NCB; ++n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              ds += tmp[n][i] * EL::to_f32(qv[rb][n][i]);
              acc[rb][n][i] += wl * tmp[n][i];
            }
          }
          ds += __shfl_xor(ds, 16, 64);
          ds += __shfl_xor(ds, 32, 64);
          if (lq == 0) inter[(w * NI + (lv - LOG2C - 1)) * C + r] = wq * ds;
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if constexpr (NT) {
        static_assert(NPRE == 2, "two buffers: the node in use and the next one");
        for (int base = 0; base < n_lev; base += 2) {
          if (base + 1 < n_lev) load_node(base + 1, nf[1]);   // gathered while this level is contracted
          contract(base, nf[0]);
          if (base + 1 >= n_lev) break;
          if (base + 2 < n_lev) load_node(base + 2, nf[0]);
          contract(base + 1, nf[1]);
        }
      } else {
        for (int base = 0; base < n_lev; base += NPRE) {
#pragma unroll
          for (int u = 0; u < NPRE; ++u) {
            const int li = base + u;
            if (li >= n_lev) break;
            contract(li, nf[u]);
            if (li + NPRE < n_lev) load_node(li + NPRE, nf[u]);
          }
        }
      }
#pragma unroll
      for (int rb = 0; rb < QB; ++rb) {
        const int r = 16 * rb + lr;
        if (r < nv) {
          E* o = reinterpret_cast<E*>(a.dq) + (bh * T + tc + r) * D + 4 * lq;
#pragma unroll
          for (int n = 0; n < NCB; ++n) store4<BF16>(o + 16 * (cb0 + n), acc[rb][n]);
        }
      }
    }
  } else {
    // ---- key side: levels whose upper block lies above the chunk
    bool act = false;
    int64_t off = 0;
    int dst_x = 0;
    int64_t xg = 0;
    if (lane >= 1 && lane <= LOG2G) {
      const int j = lane;
      if (!((ci >> (j - 1)) & 1)) {
        const int x = ((ci >> j) << j) + (1 << (j - 1));
        if (cg0 + x < nc) {
          act = true;
          off = (bh * nc + cg0 + x) * D * D;
          dst_x = x;
        }
      }
    }
    if (lane >= 32 && lane < 63) {
      const int i = lane - 31;
      if (!((gam >> (i - 1)) & 1)) {
        xg = ((gam >> i) << i) + (1ll << (i - 1));
        if (xg < ng) {
          act = true;
          off = (bh * ng + xg) * D * D;
        }
      }
    }
    const unsigned long long lmask = __ballot(act);
    const int n_lev = __popcll(lmask);
    const int pos = __popcll(lmask & ((1ull << lane) - 1ull));
    const int ent = __builtin_amdgcn_ds_permute((act ? pos : 63) << 2, lane);
    auto node_off = [&](int li, int& el) {
      el = __builtin_amdgcn_readlane(ent, li);
      const uint64_t o64 = (uint64_t)off;
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)o64, el);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(o64 >> 32), el);
      return (int64_t)(((uint64_t)hi << 32) | lo);
    };
    // node of entry li; its rows (d_k) of this wave's columns as fragments,
    // and the rows of R^T (d_v) gathered from the columns of R
    auto node_ptr = [&](int li) {
      int el;
      const int64_t o = node_off(li, el);
      return (el >= 32 ? reinterpret_cast<const E*>(a.rnodes) : reinterpret_cast<const E*>(a.rnodes_in)) + o;
    };
    auto load_rows = [&](const E* R, Frag (&rf)[KSD][NCB]) {
#pragma unroll
      for (int s2 = 0; s2 < KSD; ++s2) {
        const int k0 = s2 * KST + lq * KPL;
#pragma unroll
        for (int n = 0; n < NCB; ++n) rf[s2][n] = EL::template load_k<D>(R + (16 * (cb0 + n) + lr) * D + k0, k0);
      }
    };
    auto gather_cols = [&](const E* R, Frag (&rt)[KSD][NCB]) {
#pragma unroll
      for (int s2 = 0; s2 < KSD; ++s2) {
        const int k0 = s2 * KST + lq * KPL;
#pragma unroll
        for (int n = 0; n < NCB; ++n) rt[s2][n] = gather_node_col<BF16, D>(R, k0, 16 * (cb0 + n) + lr);
      }
    };
    float g2 = 0.f;                               // log2 gate from the chunk end to the block start
    if (nc > 1) {
      const float gx = (lane < G && cg0 + lane < nc) ? a.gch[bh * nc + cg0 + lane] : 0.f;
      const float incl = wave_incl_scan(gx);
      float S = __shfl_up(incl, 1, 64);           // S(y): gates of the group's chunks before y
      if (lane == 0) S = 0.f;
      const float after = __shfl(S, ci + 1, 64);
      const float at_x = __shfl(S, dst_x, 64);
      const float at_end = __shfl(S, G, 64);
      if (act) {
        if (lane >= 32) {
          const double* gp = a.gprefix + bh * (ng + 1);
          g2 = (at_end - after) + (float)(gp[xg] - gp[gam + 1]);
        } else {
          g2 = at_x - after;
        }
      }
    }
    if (owner) {
      Frag rf[KSD][NCB];                         // rows of the next level's node, loaded ahead
      if (n_lev > 0) load_rows(node_ptr(0), rf);
      f32x4 ak[QB][NCB], av[QB][NCB];
#pragma unroll
      for (int kb = 0; kb < QB; ++kb)
#pragma unroll
        for (int n = 0; n < NCB; ++n) ak[kb][n] = av[kb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      // dk = dS^T Q and dv = P^T dout: columns of Q and of dout as the A operand
#pragma unroll
      for (int side = 0; side < 2; ++side) {
        const unsigned char* X = side == 0 ? Qt : Gt;
        const E* SS = side == 0 ? S1 : S2;
        Frag ft[KSC][NCB];
#pragma unroll
        for (int s = 0; s < KSC; ++s)
#pragma unroll
          for (int n = 0; n < NCB; ++n)
            ft[s][n] = fused_col<BF16, C, D, DIR>(X, lay.ld_row, s * KST, 16 * (cb0 + n), lane);
#pragma unroll
        for (int kb = 0; kb < QB; ++kb) {
#pragma unroll
          for (int s = 0; s < KSC; ++s) {
            if (s * KST + KST <= 16 * kb) continue;
            const int k0 = s * KST + lq * KPL;
            Frag sf = zero_frag<BF16>();
            if (k0 < C && k0 / 16 >= kb) sf = EL::load(SS + (16 * kb + lr) * lay.ld_s + k0);
#pragma unroll
            for (int n = 0; n < NCB; ++n) {
              if (side == 0) ak[kb][n] = EL::mma(ft[s][n], sf, ak[kb][n]);
              else av[kb][n] = EL::mma(ft[s][n], sf, av[kb][n]);
            }
          }
        }
      }
      // per level: dk += gate R v over all row blocks (the R^T gathers of the
      // level in flight), the next level's rows loaded, then dv += gate R^T k;
      // each accumulator takes its terms in the order of the split kernel
      for (int li = 0; li < n_lev; ++li) {
        const E* R = node_ptr(li);
        Frag rt[KSD][NCB];
        gather_cols(R, rt);
        const int el = __builtin_amdgcn_readlane(ent, li);
        const float f = __builtin_amdgcn_exp2f(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g2), el)));
#pragma unroll
        for (int kb = 0; kb < QB; ++kb) {
          const int skr = 16 * kb + lr;
          f32x4 tk[NCB];
#pragma unroll
          for (int n = 0; n < NCB; ++n) tk[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s2 = 0; s2 < KSD; ++s2) {
            const int k0 = s2 * KST + lq * KPL;
            const auto vf = fused_row<BF16, D, DIR>(Vt, lay.ld_row, skr, k0);
#pragma unroll
            for (int n = 0; n < NCB; ++n) tk[n] = EL::mma(rf[s2][n], vf, tk[n]);
          }
          const float wk = f * e2c[skr];
#pragma unroll
          for (int n = 0; n < NCB; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) ak[kb][n][i] += wk * tk[n][i];
          __builtin_amdgcn_sched_barrier(0);
        }
        if (li + 1 < n_lev) load_rows(node_ptr(li + 1), rf);
#pragma unroll
        for (int kb = 0; kb < QB; ++kb) {
          const int skr = 16 * kb + lr;
          f32x4 tv[NCB];
#pragma unroll
          for (int n = 0; n < NCB; ++n) tv[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s2 = 0; s2 < KSD; ++s2) {
            const int k0 = s2 * KST + lq * KPL;
            const auto kf = fused_row<BF16, D, DIR>(Kt, lay.ld_row, skr, k0);
#pragma unroll
            for (int n = 0; n < NCB; ++n) tv[n] = EL::mma(rt[s2][n], kf, tv[n]);
          }
          const float wk = f * e2c[skr];
#pragma unroll
          for (int n = 0; n < NCB; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) av[kb][n][i] += wk * tv[n][i];
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // this wave's share of v_s . dv_s, then the rows of dk and dv
#pragma unroll
      for (int kb = 0; kb < QB; ++kb) {
        const int skr = 16 * kb + lr;
        float cs = 0.f;
#pragma unroll
        for (int n = 0; n < NCB; ++n) {
          const E* vrow = fused_quad<BF16, D, DIR>(Vt, lay.ld_row, skr, 16 * (cb0 + n) + 4 * lq);
#pragma unroll
          for (int i = 0; i < 4; ++i) cs += av[kb][n][i] * EL::to_f32(vrow[i]);
        }
        cs += __shfl_xor(cs, 16, 64);
        cs += __shfl_xor(cs, 32, 64);
        if (lq == 0) colS[w * C + skr] = cs;
        if (skr < nv) {
          E* okr = reinterpret_cast<E*>(a.dk) + (bh * T + tc + skr) * D + 4 * lq;
          E* ovr = reinterpret_cast<E*>(a.dv) + (bh * T + tc + skr) * D + 4 * lq;
#pragma unroll
          for (int n = 0; n < NCB; ++n) {
            store4<BF16>(okr + 16 * (cb0 + n), ak[kb][n]);
            store4<BF16>(ovr + 16 * (cb0 + n), av[kb][n]);
          }
        }
      }
    }
  }
  __syncthreads();
  if (qside) {
    // lambda gradients of the chunk's rows (as in bwd_chunk_dq): levels 0..4
    // from the diagonal tiles, 5..log2 C from the earlier tiles of the row
    // block, the rest from the query-side waves' shares; four threads per row
    const int r = tid >> 2, part = tid & 3;
    const int per = (L + 3) >> 2;
    const int rb = r >> 4, rr = r & 15;
    float rt = 0.f;
    float* dl = a.dlam + (bh * T + tc + r) * L;
    if (r < C) {
      for (int lv = part * per; lv < L && lv < (part + 1) * per; ++lv) {
        float val = 0.f;
        if (lv <= 4 && lv <= LOG2C) {
          val = partD[(rb * 16 + rr) * 5 + lv];
        } else if (lv <= LOG2C) {
          for (int kb = 0; kb < rb; ++kb)
            if (5 + (31 - __builtin_clz((unsigned)(rb ^ kb))) == lv) val += partO[(rb * (rb + 1) / 2 + kb) * 16 + rr];
        } else if ((occm >> lv) & 1u) {
          for (int u = 0; u < SH::NWA; ++u) val += inter[(u * NI + (lv - LOG2C - 1)) * C + r];
        }
        rt += lamS[r * L + lv] * val;
        if (r < nv) dl[lv] = val;
      }
    }
    rt += __shfl_xor(rt, 1, 64);
    rt += __shfl_xor(rt, 2, 64);
    if (r < nv && part == 0) a.dlog_a[bh * T + tc + r] = rt;
  } else {
    const int t = tid - 64 * NW;
    if (t < nv) {
      float cs = 0.f;
      for (int u = 0; u < SH::NWA; ++u) cs += colS[u * C + t];
      a.dcol[bh * T + tc + t] = cs;
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_gate_grad: one workgroup of 1024 threads per (b,h).  dlog_a_r =
// sum_{u >= r} (row_u - col_u), in passes of 16384 tokens from the end, read
// as 16 rows of 1024 consecutive tokens (thread t takes token t of every row:
// coalesced loads, all issued at once).  Each wave's 64 tokens of a row are
// summed from the right by shuffles in float; the 16 x 16 segment totals are
// scanned in float64 (each row by one thread, then the rows by one thread),
// and a float64 carry runs across passes.  (A template only so that every
// translation unit including this header may instantiate it.)
template <int TILE_THREADS>
__global__ __launch_bounds__(TILE_THREADS) void bwd_gate_grad(BwdArgs a) {
  static_assert(TILE_THREADS == 1024, "16 waves, 16 rows of 1024 tokens");
  constexpr int NWV = TILE_THREADS / 64, ROWS = 16, SPAN = ROWS * TILE_THREADS;
  __shared__ double seg[ROWS][NWV];     // segment totals, then the sum of the later segments of the row
  __shared__ double rtot[ROWS];         // row totals
  __shared__ double rsuf[ROWS + 1];     // sum of the later rows; [ROWS]: the pass total
  const int64_t bh = blockIdx.x, T = a.T;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  float* dl = a.dlog_a + bh * T;
  const float* dc = a.dcol + bh * T;
  double carry = 0.0;
  for (int64_t hi = T; hi > 0; hi -= SPAN) {
    const int64_t lo = hi - SPAN;                  // may be negative: the first pass is partial
    float x[ROWS];
#pragma unroll
    for (int u = 0; u < ROWS; ++u) {
      const int64_t i = lo + (int64_t)u * TILE_THREADS + tid;
      x[u] = (i >= 0 && i < hi) ? dl[i] - dc[i] : 0.f;
    }
    float sc[ROWS];                                // this token and the later ones of its wave's segment
#pragma unroll
    for (int u = 0; u < ROWS; ++u) {
      float v = x[u];
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_down(v, d, 64);
        if (lane + d < 64) v += y;
      }
      sc[u] = v;
      if (lane == 0) seg[u][w] = (double)v;
    }
    __syncthreads();
    if (tid < ROWS) {
      double acc = 0.0;
      for (int ww = NWV - 1; ww >= 0; --ww) {
        const double t = seg[tid][ww];
        seg[tid][ww] = acc;
        acc += t;
      }
      rtot[tid] = acc;
    }
    __syncthreads();
    if (tid == 0) {
      double acc = 0.0;
      for (int uu = ROWS - 1; uu >= 0; --uu) {
        rsuf[uu] = acc;
        acc += rtot[uu];
      }
      rsuf[ROWS] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < ROWS; ++u) {
      const int64_t i = lo + (int64_t)u * TILE_THREADS + tid;
      if (i >= 0 && i < hi) dl[i] = (float)(carry + rsuf[u] + seg[u][w] + (double)sc[u]);
    }
    carry += rsuf[ROWS];
    __syncthreads();                               // the shared sums are rewritten by the next pass
  }
}

// ---------------------------------------------------------------------------
// Host-side launch for one (dtype, C, D) instantiation.  fa carries the
// forward-structure buffers over (k := v, v := k).
// saved: the query-side nodes and gates are those of the caller's forward
// pass (fa and a point at its workspace), so the forward structure is not
// built again; only where the fused per-chunk kernel runs.
template <bool BF16, int C, int D>
int launch_bwd_impl(const BwdPlan& P, FwdArgs fa, BwdArgs a, hipStream_t s, bool saved) {
  using E = typename Elem<BF16>::T;
  const FwdPlan& p = P.f;
  constexpr int G = state_group(D);
  if (p.G != G) return kEHIP;
  constexpr bool kFusedShape = bwd_fused_shape(BF16, C, D);
  const bool fused = kFusedShape && P.lds_fused > 0;
  if (saved && !fused) return kEINVAL;
  bool ok = true;
  if (p.n_chunks > 1 && !saved) {
    constexpr int lds_s = state_lds(C, D, sizeof(E), G).total;
    ok = ok && hipFuncSetAttribute((const void*)fwd_chunk_states<BF16, C, D>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds_s) == hipSuccess;
    if (!ok) return kEHIP;
    hipLaunchKernelGGL((fwd_chunk_states<BF16, C, D>), dim3((unsigned)(p.n_groups * p.BH)),
                       dim3(StateShape<BF16, C, D>::NT), lds_s, s, fa);
    ok = ok && hipGetLastError() == hipSuccess;
  }
  if (p.n_groups > 1 && !saved) {
    const dim3 grid((unsigned)(group_tree_blocks(D) * p.BH));
    const int levels = bit_length(p.n_groups);
    if (levels <= 6)
      hipLaunchKernelGGL((fwd_group_tree<BF16, 6>), grid, dim3(kTreeThreads), 0, s, fa, D);
    else if (levels <= 8)
      hipLaunchKernelGGL((fwd_group_tree<BF16, 8>), grid, dim3(kTreeThreads), 0, s, fa, D);
    else if (levels <= 16)
      hipLaunchKernelGGL((fwd_group_tree<BF16, 16>), grid, dim3(kTreeThreads), 0, s, fa, D);
    else
      hipLaunchKernelGGL((fwd_group_tree<BF16, 32>), grid, dim3(kTreeThreads), 0, s, fa, D);
    ok = ok && hipGetLastError() == hipSuccess;
  }
  // the fused per-chunk kernel needs the key-side nodes first; the query-side
  // kernel of the split pair does not
  if (!fused) {
    ok = ok && hipFuncSetAttribute((const void*)bwd_chunk_dq<BF16, C, D>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, P.lds_dq) == hipSuccess;
    if (!ok) return kEHIP;
    hipLaunchKernelGGL((bwd_chunk_dq<BF16, C, D>), dim3((unsigned)(p.n_chunks * p.BH)), dim3(64 * bwd_waves(C)),
                       P.lds_dq, s, a);
    ok = ok && hipGetLastError() == hipSuccess;
  }
  if (p.n_chunks > 1) {
    if constexpr (rev_cm_fits(BF16, C, D, G)) {
      constexpr int lds = rev_cm_lds(C, D, G).total;
      ok = ok && hipFuncSetAttribute((const void*)bwd_rev_states_cm<C, D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess;
      if (!ok) return kEHIP;
      hipLaunchKernelGGL((bwd_rev_states_cm<C, D>), dim3((unsigned)(2 * p.n_groups * p.BH)),
                         dim3(64 * state_waves(D)), lds, s, a);
    } else if constexpr (rev_staged_fits(BF16, C, D, G)) {
      constexpr int lds = rev_staged_lds(C, D, G).total;
      ok = ok && hipFuncSetAttribute((const void*)bwd_rev_states_staged<C, D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess;
      if (!ok) return kEHIP;
      hipLaunchKernelGGL((bwd_rev_states_staged<C, D>), dim3((unsigned)(2 * p.n_groups * p.BH)),
                         dim3(64 * state_waves(D)), lds, s, a);
    } else {
      ok = ok && hipFuncSetAttribute((const void*)bwd_rev_states<BF16, C, D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, P.lds_rev) == hipSuccess;
      if (!ok) return kEHIP;
      hipLaunchKernelGGL((bwd_rev_states<BF16, C, D>), dim3((unsigned)(p.n_groups * p.BH)),
                         dim3(64 * state_waves(D)), P.lds_rev, s, a);
    }
    ok = ok && hipGetLastError() == hipSuccess;
  }
  if (p.n_groups > 1) {
    hipLaunchKernelGGL((bwd_rev_tree<BF16>), dim3((unsigned)(p.BH * (p.n_groups - 1) * (D / 16))), dim3(256), 0, s, a,
                       D);
    ok = ok && hipGetLastError() == hipSuccess;
  }
  if constexpr (kFusedShape) {
    if (fused && saved) {
      ok = ok && hipFuncSetAttribute((const void*)bwd_chunk_fused<BF16, C, D, true>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, P.lds_fused) == hipSuccess;
      if (!ok) return kEHIP;
      hipLaunchKernelGGL((bwd_chunk_fused<BF16, C, D, true>), dim3((unsigned)(p.n_chunks * p.BH)),
                         dim3(128 * bwd_waves(C)), P.lds_fused, s, a);
      ok = ok && hipGetLastError() == hipSuccess;
    } else if (fused) {
      ok = ok && hipFuncSetAttribute((const void*)bwd_chunk_fused<BF16, C, D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, P.lds_fused) == hipSuccess;
      if (!ok) return kEHIP;
      hipLaunchKernelGGL((bwd_chunk_fused<BF16, C, D>), dim3((unsigned)(p.n_chunks * p.BH)),
                         dim3(128 * bwd_waves(C)), P.lds_fused, s, a);
      ok = ok && hipGetLastError() == hipSuccess;
    }
  }
  if (!fused) {
    ok = ok && hipFuncSetAttribute((const void*)bwd_chunk_dkv<BF16, C, D>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, P.lds_dkv) == hipSuccess;
    if (!ok) return kEHIP;
    hipLaunchKernelGGL((bwd_chunk_dkv<BF16, C, D>), dim3((unsigned)(p.n_chunks * p.BH)), dim3(64 * bwd_waves(C)),
                       P.lds_dkv, s, a);
    ok = ok && hipGetLastError() == hipSuccess;
  }
  hipLaunchKernelGGL((bwd_gate_grad<1024>), dim3((unsigned)p.BH), dim3(1024), 0, s, a);
  ok = ok && hipGetLastError() == hipSuccess;
  return ok ? kOK : kEHIP;
}

template <bool BF16>
int launch_bwd_dtype(const BwdPlan& P, const FwdArgs& fa, const BwdArgs& a, hipStream_t s, bool saved) {
#define LA_CASE(CC, DD) \
  if (P.f.C == CC && P.f.D == DD) return launch_bwd_impl<BF16, CC, DD>(P, fa, a, s, saved);
  LA_CASE(16, 16) LA_CASE(16, 32) LA_CASE(16, 64) LA_CASE(16, 128)
  LA_CASE(32, 16) LA_CASE(32, 32) LA_CASE(32, 64) LA_CASE(32, 128)
  LA_CASE(64, 16) LA_CASE(64, 32) LA_CASE(64, 64) LA_CASE(64, 128)
#undef LA_CASE
  return kESHAPE;
}

}  // namespace la
