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
// so the levels above c form a Fenwick tree over chunks.  Every bucket of
// that tree is an aligned block of 2^(j-1) chunks; the bucket a query chunk
// needs at chunk level j is the block ending at chunk
//   e = ((chunk >> j) << j) + 2^(j-1) - 1,
// i.e. the block of 2^ctz(e+1) chunks that ends at e.  So one node per chunk,
// "the bucket ending here", holds every bucket any query needs.
//
// Three kernels build and use those nodes:
//   fwd_chunk_states  per group of G = 2^g chunks: the chunk states
//                     K_c^T diag(gate) V_c on the matrix cores, merged with
//                     the binary-counter carry of the decode recurrence
//                     (held in registers); writes the node of every chunk
//                     whose bucket stays inside the group (levels c+1..c+g)
//                     and the group's aggregate state
//   fwd_group_tree    per (b,h): the same carry over groups, writing the node
//                     of every group (levels above c+g) and float64 prefix
//                     sums of the group gate totals
//   fwd_chunk_output  per chunk: the masked C x C score tile, its product with
//                     V, and one contraction per occupied level with the
//                     lambda- and gate-weighted queries; writes the output.
// Gates are carried in log2 units (log_a * log2 e); the gates applied are
// products of a_r <= 1, so every exponent is <= 0.  Sums inside a chunk are
// float32; gate sums across groups are float64.
#pragma once

#include "la_device.hpp"
#include "la_levels.hpp"
#include "la_plan.hpp"

namespace la {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_a;
  const float* lam;
  void* out;
  void* nodes_in;     // [BH][n_chunks][D][D] element type, (d_v, d_k) order: bucket ending at a chunk
  float* gch;         // [BH][n_chunks] log2 gate total of each chunk
  float* gstate;      // [BH][n_groups][D][D] fp32, (d_v, d_k) order: whole-group state
  float* gtot;        // [BH][n_groups] log2 gate total of each group
  double* gprefix;    // [BH][n_groups + 1] exclusive prefix sums of gtot
  void* nodes;        // [BH][n_groups][D][D] element type: bucket ending at a group
  int64_t T;
  int64_t n_chunks;
  int64_t n_groups;
  int64_t n_full_groups;  // groups of G chunks of C tokens each
  int L;
  int lam_vec4;           // lambda rows of every full chunk are 16-byte aligned
  // heads per q/k head group: q and k are [B][H / qk_div][T][d] and head h
  // reads group h / qk_div (a layer whose heads share B and C); 0 or 1: one
  // q and k per head
  int qk_div;
  // final recurrent state (loglinear_fwd_state): [BH][st_S][D][D] fp32 slots
  // and [BH][st_S] scales; null when not asked for
  float* st_slots;
  float* st_scale;
  int st_S;
};

constexpr int cilog2(int x) { return x <= 1 ? 0 : 1 + cilog2(x >> 1); }

// Inclusive prefix sum of log2(a) over one chunk of C tokens starting at
// `base`, by one wave, into b2c[0..C); zero past the end of the sequence.
template <int C>
__device__ __forceinline__ void chunk_gate_scan(const float* la_bh, int64_t base, int64_t T, float* b2c) {
  const int lane = lane_id();
  if constexpr (C <= 64) {
    float x = 0.f;
    if (lane < C && base + lane < T) x = la_bh[base + lane] * kLog2e;
    x = wave_incl_scan(x);
    if (lane < C) b2c[lane] = x;
  } else {
    static_assert(C == 128, "chunk sizes above 64 must be 128");
    const int64_t i0 = base + 2 * lane;
    const float x0 = i0 < T ? la_bh[i0] * kLog2e : 0.f;
    const float x1 = i0 + 1 < T ? la_bh[i0 + 1] * kLog2e : 0.f;
    const float s = wave_incl_scan(x0 + x1);
    b2c[2 * lane] = s - x1;
    b2c[2 * lane + 1] = s;
  }
}

// Column swizzle of the transposed (token-contiguous) tiles of the state
// kernel: row n's tokens are XOR-permuted in granules of 8 by its 8-row block,
// masked to the chunk width.
template <int C>
__device__ __forceinline__ int state_swz(int n) { return 8 * ((n >> 3) & (C / 8 - 1)); }

// ---------------------------------------------------------------------------
// fwd_chunk_states: one workgroup per (b,h, group of G chunks).
template <bool BF16, int C, int D>
struct StateShape {
  using EL = Elem<BF16>;
  static constexpr int NW = state_waves(D), NT = 64 * NW;
  static constexpr int DB = D / 16, HT = DB * DB, TPW = state_tiles_per_wave(D);
  static constexpr int G = state_group(D);
  static constexpr int NS = cilog2(G) > 0 ? cilog2(G) : 1;
  static constexpr int KSC = (C + EL::kStep - 1) / EL::kStep;
  static constexpr int EPV = 16 / (BF16 ? 2 : 4), VPR = D / EPV, NV = C * VPR;
  static constexpr int NPF = (NV + NT - 1) / NT;
};

template <bool BF16, int C, int D>
__global__ __launch_bounds__(64 * state_waves(D)) void fwd_chunk_states(FwdArgs a) {
  using SH = StateShape<BF16, C, D>;
  using EL = Elem<BF16>;
  using E = typename EL::T;
  constexpr int G = SH::G, NS = SH::NS, DB = SH::DB, TPW = SH::TPW, NW = SH::NW;
  constexpr int KPL = EL::kPerLane, KST = EL::kStep, EPV = SH::EPV;
  constexpr StateLds lay = state_lds(C, D, sizeof(E), G);
  extern __shared__ __align__(16) unsigned char smem[];
  float* b2s = reinterpret_cast<float*>(smem + lay.b2);

  const int64_t ng = a.n_groups, nc = a.n_chunks;
  const int64_t bh = blockIdx.x / ng;
  const int64_t gam = blockIdx.x % ng;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id(), lq = lane >> 4, lr = lane & 15;
  const int64_t T = a.T;
  const int64_t c0 = gam * G;
  const int nch = (int)(nc - c0 < G ? nc - c0 : G);
  const int64_t t0 = c0 * C;
  const float* la_bh = a.log_a + bh * T;
  const int64_t kbh = a.qk_div > 1 ? bh / a.qk_div : bh;   // k's head (group)
  const E* kb = reinterpret_cast<const E*>(a.k) + (kbh * T + t0) * D;
  const E* vb = reinterpret_cast<const E*>(a.v) + (bh * T + t0) * D;
  uint4 pk[2][SH::NPF], pv[2][SH::NPF];
  auto prefetch = [&](int c, uint4 (&dk)[SH::NPF], uint4 (&dv)[SH::NPF]) {
    const int nv = (int)(T - t0 - (int64_t)c * C < C ? T - t0 - (int64_t)c * C : C);
#pragma unroll
    for (int p = 0; p < SH::NPF; ++p) {
      const int idx = tid + p * SH::NT;
      const int r = idx / SH::VPR, cv = idx % SH::VPR;   // columns fastest: each row read whole
      dk[p] = dv[p] = make_uint4(0, 0, 0, 0);
      if (idx < SH::NV && r < nv) {
        const int64_t off = ((int64_t)c * C + r) * D + cv * EPV;
        dk[p] = *reinterpret_cast<const uint4*>(kb + off);
        dv[p] = *reinterpret_cast<const uint4*>(vb + off);
      }
    }
  };
  // the first two chunks load while the gates are scanned
  prefetch(0, pk[0], pv[0]);
  if (nch > 1) prefetch(1, pk[1], pv[1]);
  for (int c = w; c < nch; c += NW) chunk_gate_scan<C>(la_bh, t0 + (int64_t)c * C, T, b2s + c * C);
  __syncthreads();

  float gch[G];
  float gt = 0.f;
#pragma unroll
  for (int c = 0; c < G; ++c) {
    gch[c] = c < nch ? b2s[c * C + C - 1] : 0.f;
    gt += gch[c];
  }
  if (tid < nch) a.gch[bh * nc + c0 + tid] = b2s[tid * C + C - 1];
  if (tid == 0 && (gam + 1) * G * C <= T) a.gtot[bh * ng + gam] = gt;

  f32x4 sl[NS][TPW];   // in-group carry: bucket states of levels 1..NS, fp32
  float sc2[NS];       // their lazy log2 gates (from the bucket end to the current chunk start)
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    sc2[j] = 0.f;
#pragma unroll
    for (int h = 0; h < TPW; ++h) sl[j][h] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  E* nin = reinterpret_cast<E*>(a.nodes_in) + (bh * nc + c0) * D * D;

#pragma unroll
  for (int c = 0; c < G; ++c) {
    if (c >= nch) break;
    float gc = 0.f;
#pragma unroll
    for (int u = 0; u < G; ++u) gc = (u == c) ? gch[u] : gc;
    const float* b2c = b2s + c * C;
    // this chunk's buffer (selects, not indexing: the layout stays in registers)
    E* VT = reinterpret_cast<E*>(smem + ((c & 1) ? lay.vt[1] : lay.vt[0]));
    E* KTs = reinterpret_cast<E*>(smem + ((c & 1) ? lay.kts[1] : lay.kts[0]));
    // stage V^T and K^T gated to the chunk end (with one buffer, the previous
    // chunk's readers must be done first).  A lane holds EPV elements of one
    // token row; the column (token) of row n is XOR-swizzled in 8-token
    // granules by swz(n), so the lanes writing the rows of one granule of d
    // land in different banks, and a fragment read stays one whole granule.
    if (lay.nbuf == 1 && c > 0) __syncthreads();
#pragma unroll
    for (int p = 0; p < SH::NPF; ++p) {
      const int idx = tid + p * SH::NT;
      if (idx < SH::NV) {
        const int r = idx / SH::VPR, cv = idx % SH::VPR;
        const E* ke = reinterpret_cast<const E*>(&pk[c & 1][p]);
        const E* ve = reinterpret_cast<const E*>(&pv[c & 1][p]);
        const float u = __builtin_amdgcn_exp2f(gc - b2c[r]);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int n = cv * EPV + e;
          const int col = r ^ state_swz<C>(n);
          VT[n * lay.ld_t + col] = ve[e];
          KTs[n * lay.ld_t + col] = EL::from_f32(EL::to_f32(ke[e]) * u);
        }
      }
    }
    __syncthreads();
    if (c + 2 < nch) prefetch(c + 2, pk[c & 1], pv[c & 1]);

    int kk = 0;                                   // trailing ones of c
    for (int x = c; x & 1; x >>= 1) ++kk;
    float fj[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) fj[j] = j < kk ? __builtin_amdgcn_exp2f(sc2[j] + gc) : 0.f;
    const int64_t cg = c0 + c;
    // the bucket ending at every full chunk, and every full group's state
    const bool write_node = (c != G - 1) && ((cg + 1) * C <= T);
    const bool write_group = (c == G - 1) && ((gam + 1) * G * C <= T);
#pragma unroll
    for (int h = 0; h < TPW; ++h) {
      const int tix = w + h * NW;
      if (tix >= SH::HT) continue;
      const int mb = tix / DB, nb = tix % DB;
      // transposed tile: hh[i] = H[d_v = 16 mb + lr][d_k = 16 nb + 4 lq + i]
      f32x4 hh = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < SH::KSC; ++s) {
        const int k0 = s * KST + lq * KPL;
        const int nv_ = 16 * mb + lr, nk_ = 16 * nb + lr;
        const auto va = EL::template load_k<C>(VT + nv_ * lay.ld_t + (k0 ^ state_swz<C>(nv_)), k0);
        const auto kf = EL::template load_k<C>(KTs + nk_ * lay.ld_t + (k0 ^ state_swz<C>(nk_)), k0);
        hh = EL::mma(kf, va, hh);
      }
      // the bucket ending at this chunk: the chunk plus levels 1..kk
#pragma unroll
      for (int j = 0; j < NS; ++j)
        if (j < kk) hh += fj[j] * sl[j][h];
      {
        const int row = 16 * mb + lr, col = 16 * nb + 4 * lq;      // (d_v, d_k .. d_k + 3)
        if (write_node) {
          E* o = nin + (int64_t)c * D * D + row * D + col;
          if constexpr (BF16)
            *reinterpret_cast<u16x4*>(o) = u16x4{f32_to_bf16(hh[0]), f32_to_bf16(hh[1]), f32_to_bf16(hh[2]),
                                                 f32_to_bf16(hh[3])};
          else
            *reinterpret_cast<f32x4*>(o) = hh;
        }
        if (write_group) *reinterpret_cast<f32x4*>(a.gstate + (bh * ng + gam) * D * D + row * D + col) = hh;
      }
#pragma unroll
      for (int j = 0; j < NS; ++j)
        if (j == kk) sl[j][h] = hh;
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) sc2[j] = (j == kk) ? 0.f : sc2[j] + gc;
    // with two buffers the next chunk is staged into the other one, which
    // was last read before this chunk's barrier
  }
}

// ---------------------------------------------------------------------------
// Group tree: per (b,h) and kTreeVec consecutive state elements, walk the
// full groups with the binary-counter carry.  node[e] = A_e + sum_{j<=k} gate * bucket_j where
// k = trailing ones of e: the bucket of 2^k groups ending at group e.  It
// also writes gprefix[0 .. n_full_groups], the exclusive prefix sums of the
// group gate totals.  MAXJ bounds the carry levels (bit length of the group
// count); the launcher picks the smallest instantiation that covers the
// sequence.
// Workgroups of kTreeThreads threads per (b,h), kTreeVec consecutive state
// elements (one 16-byte load per group) per thread.
constexpr int kTreeVec = 4;   // consecutive state elements per thread of the group tree
constexpr int kTreeThreads = 256;
typedef float ftv __attribute__((ext_vector_type(kTreeVec)));
typedef unsigned short utv __attribute__((ext_vector_type(kTreeVec)));
LA_HD constexpr int group_tree_blocks(int D) { return (D * D / kTreeVec + kTreeThreads - 1) / kTreeThreads; }

template <bool BF16, int MAXJ>
__global__ __launch_bounds__(kTreeThreads) void fwd_group_tree(FwdArgs a, int D) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  constexpr int V = kTreeVec;   // consecutive state elements per thread: one vector load per group
  const int DD = D * D, NQ = DD / V;
  const int nblk = group_tree_blocks(D);
  const int64_t bh = blockIdx.x / nblk;
  const int blk = blockIdx.x % nblk;
  const int q4 = blk * kTreeThreads + threadIdx.x;
  const bool valid = q4 < NQ;
  const int64_t ng = a.n_groups, nfg = a.n_full_groups;
  ftv slot[MAXJ];
  float fac[MAXJ];    // gate product from the end of slot j's bucket to the current group
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) { slot[j] = ftv(0.f); fac[j] = 1.f; }
  double pre = 0.0;
  const bool writer = blk == 0 && threadIdx.x == 0;
  const ftv* gs = reinterpret_cast<const ftv*>(a.gstate + bh * ng * DD);
  E* nd = reinterpret_cast<E*>(a.nodes) + bh * ng * DD;
  // groups are walked in batches of kBatch; the loads of the next batch are
  // issued before the current one is walked (two register buffers, the batch
  // loop unrolled by two so that both buffers keep constant indices; macros
  // rather than lambdas, which would send the arrays to scratch memory).
  // Short walks (under 64 groups) reach their first node sooner with batches
  // of 4 (16K tokens at d = 64: 21.1 -> 20.7 us); long ones stream better
  // with 8 (128K tokens at d = 128: 82 us, against 91 with 4).
  constexpr int kBatch = MAXJ <= 6 ? 4 : 8;
  ftv A0[kBatch], A1[kBatch];
  float g0[kBatch], g1[kBatch];
#define LA_TREE_LOAD(E0, Av, gv)                          \
  do {                                                    \
    _Pragma("unroll") for (int u = 0; u < kBatch; ++u) {  \
      const int64_t e = (E0) + u;                         \
      Av[u] = ftv(0.f);                                   \
      gv[u] = 0.f;                                        \
      if (e < nfg) {                                      \
        gv[u] = a.gtot[bh * ng + e];                      \
        if (valid) Av[u] = gs[e * NQ + q4];               \
      }                                                   \
    }                                                     \
  } while (0)
  // node[e] = A_e + sum over the k = trailing-ones(e) lower slots, decayed
  // to e; e0 is a multiple of kBatch, so for u < kBatch - 1 the trailing ones
  // are those of u (a constant of the unrolled loop: the slot updates resolve
  // at compile time); the last group of a batch continues into e0 / kBatch
#define LA_TREE_WALK(E0, Av, gv)                                                                         \
  do {                                                                                                   \
    _Pragma("unroll") for (int u = 0; u < kBatch; ++u) {                                                 \
      const int64_t e = (E0) + u;                                                                        \
      if (e >= nfg) continue;                                                                            \
      if (writer) a.gprefix[bh * (ng + 1) + e] = pre;                                                    \
      const float g = gv[u];                                                                             \
      const float eg = __builtin_amdgcn_exp2f(g);                                                        \
      const int kk = (u < kBatch - 1) ? __builtin_ctz(~(unsigned)u)                                      \
                                      : cilog2(kBatch) + __builtin_ctzll(~(unsigned long long)((E0) / kBatch)); \
      ftv nw = Av[u];                                                                                    \
      _Pragma("unroll") for (int j = 0; j < MAXJ; ++j) {                                                 \
        fac[j] *= eg;                                                                                    \
        if (j < kk) {                                                                                    \
          _Pragma("unroll") for (int i = 0; i < V; ++i) nw[i] = fmaf(fac[j], slot[j][i], nw[i]);        \
        }                                                                                                \
      }                                                                                                  \
      _Pragma("unroll") for (int j = 0; j < MAXJ; ++j) if (j == kk) { slot[j] = nw; fac[j] = 1.f; }    \
      if (valid) {                                                                                       \
        if constexpr (BF16) {                                                                            \
          utv o;                                                                                         \
          _Pragma("unroll") for (int i = 0; i < V; ++i) o[i] = EL::from_f32(nw[i]);                      \
          *reinterpret_cast<utv*>(nd + e * DD + V * q4) = o;                                             \
        } else {                                                                                         \
          *reinterpret_cast<ftv*>(nd + e * DD + V * q4) = nw;                                            \
        }                                                                                                \
      }                                                                                                  \
      pre += (double)g;                                                                                  \
    }                                                                                                    \
  } while (0)
  if (nfg > 0) LA_TREE_LOAD(0, A0, g0);
  for (int64_t e0 = 0; e0 < nfg; e0 += 2 * kBatch) {
    if (e0 + kBatch < nfg) LA_TREE_LOAD(e0 + kBatch, A1, g1);
    LA_TREE_WALK(e0, A0, g0);
    if (e0 + kBatch >= nfg) break;
    if (e0 + 2 * kBatch < nfg) LA_TREE_LOAD(e0 + 2 * kBatch, A0, g0);
    LA_TREE_WALK(e0 + kBatch, A1, g1);
  }
#undef LA_TREE_LOAD
#undef LA_TREE_WALK
  if (writer) a.gprefix[bh * (ng + 1) + nfg] = pre;
}

// ---------------------------------------------------------------------------
// fwd_final_state: the recurrent (decode) state after the T tokens, for a
// decode that continues at position T ("Log-Linear Attention", Italian
// summary, technical section 2, item 3: the recurrent form keeps one state per
// occupied level).  One block per (b,h).  Slot i holds level i+1, occupied
// iff bit i of T is set: the bucket of keys [((T >> i) << i) - 2^i,
// (T >> i) << i), each key weighted by its gate product up to token T-1, as a
// (d_k, d_v) float32 matrix with scale 1.  Buckets smaller than a chunk lie in
// the last, partial chunk and are summed here from k and v; the others are the
// node the forward built for the bucket's last chunk (levels inside a group)
// or last group, decayed from its end to token T-1.  Slots of empty levels
// are left as they are: a decode step never reads them and overwrites a slot
// whole when its level fills.
template <bool BF16, int C, int D>
__global__ __launch_bounds__(256) void fwd_final_state(FwdArgs a) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  constexpr int G = state_group(D), LOG2C = cilog2(C), LOG2G = cilog2(G);
  constexpr int DD = D * D, NQ = DD / 4, PER = (NQ + 255) / 256;   // four (d_k, d_v..d_v+3) entries per item
  __shared__ float wk[C / 2];
  const int S = a.st_S;
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t T = a.T, nc = a.n_chunks;
  if (tid < S) a.st_scale[bh * S + tid] = 1.f;
  for (int i = 0; i < S; ++i) {
    if (!((T >> i) & 1)) continue;
    const int64_t s1 = (T >> i) << i, s0 = s1 - (1ll << i);
    f32x4 acc[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < LOG2C) {
      // keys s0 .. s1-1 of the last chunk, weight exp2(sum_{r=s+1}^{T-1} log2 a_r)
      const int nk = 1 << i;
      if (tid < nk) {
        float g = 0.f;
        for (int64_t r = s0 + tid + 1; r < T; ++r) g += a.log_a[bh * T + r] * kLog2e;
        wk[tid] = __builtin_amdgcn_exp2f(g);
      }
      __syncthreads();
      const E* kb = reinterpret_cast<const E*>(a.k) + ((a.qk_div > 1 ? bh / a.qk_div : bh) * T + s0) * D;
      const E* vb = reinterpret_cast<const E*>(a.v) + (bh * T + s0) * D;
      for (int j = 0; j < nk; ++j) {
        const float wj = wk[j];
#pragma unroll
        for (int p = 0; p < PER; ++p) {
          const int e = 4 * (tid + p * 256);
          if (e < DD) {
            const float kw = wj * EL::to_f32(kb[j * D + e / D]);
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[p][u] += kw * EL::to_f32(vb[j * D + e % D + u]);
          }
        }
      }
      __syncthreads();                              // wk is read out before the next level
    } else {
      // log2 gate from the node's end to token T-1
      const bool grp = i >= LOG2C + LOG2G;
      const int64_t ce = s1 / C - 1;                  // last chunk of the bucket
      double g = 0.0;
      const E* node;
      if (grp) {
        const int64_t e = s1 / ((int64_t)C * G) - 1;  // last group of the bucket
        const double* gp = a.gprefix + bh * (a.n_groups + 1);
        g = gp[a.n_full_groups] - gp[e + 1];
        for (int64_t c = a.n_full_groups * G; c < nc; ++c) g += (double)a.gch[bh * nc + c];
        node = reinterpret_cast<const E*>(a.nodes) + (bh * a.n_groups + e) * DD;
      } else {
        for (int64_t c = ce + 1; c < nc; ++c) g += (double)a.gch[bh * nc + c];
        node = reinterpret_cast<const E*>(a.nodes_in) + (bh * nc + ce) * DD;
      }
      const float f = __builtin_amdgcn_exp2f((float)g);
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int e = 4 * (tid + p * 256);
        if (e < DD) {
          const int dk = e / D, dv = e % D;         // nodes are (d_v, d_k)
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[p][u] = f * EL::to_f32(node[(dv + u) * D + dk]);
        }
      }
    }
    float* out = a.st_slots + (bh * S + i) * DD;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = 4 * (tid + p * 256);
      if (e < DD) *reinterpret_cast<f32x4*>(out + e) = acc[p];
    }
  }
}

// ---------------------------------------------------------------------------
// fwd_chunk_output: one workgroup per (b,h, chunk).
//
// Phase 1 forms the causal score tiles S^T = K Q^T (key block kb <= query
// block qb), dealt round-robin over the waves, masks them with the gate and
// the level weight of every (query, key) pair and writes the masked tile P
// to LDS.  Phase 2 gives each wave a block of 16 output columns for all C
// query rows: O = P V, then one product Q node^T per occupied level above
// the chunk, weighted per query row by lambda and the gate.  Owning columns
// means a wave reads only its 16 rows of each (d_v, d_k) node, so every node
// crosses from L2 once per chunk.
template <bool BF16, int C, int D>
struct ChunkShape {
  using EL = Elem<BF16>;
  static constexpr int NW = output_waves(C), NT = 64 * NW;
  static constexpr int QB = C / 16, DB = D / 16;
  static constexpr int NST = QB * (QB + 1) / 2;                // causal score tiles
  static constexpr int NCB = DB > NW ? DB / NW : 1;           // column blocks per wave
  static constexpr int KSD = (D + EL::kStep - 1) / EL::kStep;  // k-steps over d
  static constexpr int KSC = (C + EL::kStep - 1) / EL::kStep;  // k-steps over keys
  static constexpr int EPV = 16 / (BF16 ? 2 : 4), VPR = D / EPV, NV = C * VPR;
  static constexpr int NPF = (NV + NT - 1) / NT;
  static constexpr int NPL = (C * kMaxLevels + NT - 1) / NT;   // lambda values per thread (bound)
  static constexpr int NPL4 = (C * kMaxLevels / 4 + NT - 1) / NT;   // ... as float4 loads
  static constexpr int NLX = NPL > 4 * NPL4 ? NPL : 4 * NPL4;   // registers for either
  // small tiles: the first NPRE levels' nodes load with the chunk; larger
  // ones load them at the start of phase 2, where the registers are free
  static constexpr bool EARLY = BF16 && C <= 64 && D <= 64;
  static constexpr int NPRE = EARLY && !output_direct(C, D, BF16 ? 2 : 4) ? 4 : 2;   // node fragment buffers per wave
};

// Direct-load tiles (bfloat16, D = 64 or 128): unpadded rows of 2 D bytes,
// the 16-byte granule g of row r stored at granule g ^ (r mod 8) of that row,
// so the 16 rows an operand fragment reads spread over the banks.  The direct
// global-to-LDS loads write whole 1 KB runs, so the permutation is applied to
// the global addresses the lanes load.
template <int D>
__device__ __forceinline__ int swz_gran(int r, int g) { return r * (2 * D) + ((g ^ (r & 7)) << 4); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposed bfloat16 fragment of a direct-load tile (ds_read_b64_tr_b16: the
// 16 lanes of a group each read 8 bytes, four consecutive columns of one of
// four rows, and lane i receives column i of the four rows): lane (lq, lr)
// receives rows k0 + 8 lq .. + 7 of column c0 + lr, the k-slice of an operand
// whose rows are the tile's columns.
// The two halves: lo holds rows k0 + 8 lq .. + 3, hi rows k0 + 8 lq + 4 .. + 7.
// Code that works on the elements takes them from the halves: extracting
// elements after a bit-cast round trip through bf16x8 was compiled as if
// every element were element 0.
template <int D>
__device__ __forceinline__ void swz_tr_halves(const unsigned char* tile, int k0, int c0, int lane, i16x4& lo,
                                              i16x4& hi) {
  const int lq = lane >> 4, j = lane & 15;
  const int g = (c0 >> 3) + ((j & 3) >> 1), o = (j & 1) * 8;
  const int r0 = k0 + 8 * lq + (j >> 2);
  lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + swz_gran<D>(r0, g) + o));
  hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + swz_gran<D>(r0 + 4, g) + o));
}
template <int D>
__device__ __forceinline__ bf16x8 swz_tr_frag(const unsigned char* tile, int k0, int c0, int lane) {
  i16x4 lo, hi;
  swz_tr_halves<D>(tile, k0, c0, lane, lo, hi);
  return __builtin_bit_cast(bf16x8, u16x8{(unsigned short)lo[0], (unsigned short)lo[1], (unsigned short)lo[2],
                                          (unsigned short)lo[3], (unsigned short)hi[0], (unsigned short)hi[1],
                                          (unsigned short)hi[2], (unsigned short)hi[3]});
}

// FULL: the chunk has C rows (every chunk but a ragged last one), so the
// row bounds checks fold away.
//
// Phase 2 works on transposed tiles: with the MFMA operands swapped
// (V^T P^T and node Q^T) a lane holds one query row and four consecutive
// output columns, so each row weight is one value per lane and each output
// row slice is one contiguous store.
//
// VL (late V): the level contractions run before P V, and V is loaded into
// the Q tile once every wave is past its Q reads, so the tiles take one buffer
// less (32 KB at C = d = 128, where that lets two workgroups share a CU; 8 KB
// at C = d = 64, seven workgroups per CU in place of five).
template <bool BF16, int C, int D, bool FULL, bool VL = false>
__device__ __forceinline__ void chunk_output_body(const FwdArgs& a, unsigned char* smem, int64_t item) {
  using SH = ChunkShape<BF16, C, D>;
  using EL = Elem<BF16>;
  using E = typename EL::T;
  using Frag = typename EL::Frag;
  constexpr int QB = SH::QB, DB = SH::DB, KSD = SH::KSD, NCB = SH::NCB, NW = SH::NW, NPRE = SH::NPRE;
  constexpr int KPL = EL::kPerLane, KST = EL::kStep, EPV = SH::EPV;
  constexpr int G = state_group(D);
  constexpr int LOG2C = cilog2(C), LOG2G = cilog2(G);
  const int L = a.L;
  const OutLds lay = VL ? output_lds_vlate(C, D, sizeof(E), L) : output_lds(C, D, sizeof(E), L);
  E* Qs = reinterpret_cast<E*>(smem + lay.q);
  E* Ks = reinterpret_cast<E*>(smem + lay.k);
  E* Vs = reinterpret_cast<E*>(smem + lay.v);
  E* Ps = reinterpret_cast<E*>(smem + lay.p);
  float* lamS = reinterpret_cast<float*>(smem + lay.lam);
  float* b2c = reinterpret_cast<float*>(smem + lay.b2);
  float* e2c = reinterpret_cast<float*>(smem + lay.e2);

  constexpr bool DIRECT = output_direct(C, D, sizeof(E));
  static_assert(!VL || (DIRECT && NW * NCB == DB), "late V: direct tiles, every wave owns output columns");
  constexpr int NTL = VL ? 2 : 3;                  // tiles loaded with the chunk: Q, K (and V)
  const unsigned char* Qt = smem + lay.q;         // direct-load tiles (swizzled rows)
  const unsigned char* Kt = smem + lay.k;
  const unsigned char* Vt = smem + lay.v;

  const int64_t nc = a.n_chunks, ng = a.n_groups;
  // B * H * n_chunks < 2^31 (checked on the host): 32-bit division
  const int64_t bh = (uint32_t)item / (uint32_t)nc;
  const int64_t c = (uint32_t)item % (uint32_t)nc;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id(), lq = lane >> 4, lr = lane & 15;
  const int64_t T = a.T;
  const int64_t tc = c * C;
  const int nv = FULL ? C : (int)(T - tc < C ? T - tc : C);

  const int64_t qkbh = a.qk_div > 1 ? bh / a.qk_div : bh;  // q's and k's head (group)
  const E* qg = reinterpret_cast<const E*>(a.q) + (qkbh * T + tc) * D;
  const E* kg = reinterpret_cast<const E*>(a.k) + (qkbh * T + tc) * D;
  const E* vg = reinterpret_cast<const E*>(a.v) + (bh * T + tc) * D;
  E* og = reinterpret_cast<E*>(a.out) + (bh * T + tc) * D;
  const float* lg = a.lam + (bh * T + tc) * L;

  // ---- loads of this chunk, all issued before the first LDS store
  uint4 qx[SH::NPF], kx[SH::NPF], vx[SH::NPF];
  float lx[SH::NLX];
  // lambda rows: 16-byte loads on full chunks when aligned, else one value
  // per load
  const bool lam4 = FULL && a.lam_vec4;
  if constexpr (DIRECT) {
    constexpr int ROWB = 2 * D, GPR = ROWB / 16, RPR = 1024 / ROWB, RUNS = C * ROWB / 1024;
    if (FULL) {
      // direct global-to-LDS loads in 1 KB runs: lane l fills granule l mod GPR
      // of row RPR ri + l / GPR with the logical granule that XORs to it.  The
      // row's low three bits are (RPR ri + l / GPR) mod 8, so the lane's source
      // offset inside a run is the same for every run when RPR >= 8 and
      // alternates with ri when RPR = 4.
      static_assert((NTL * RUNS) % NW == 0, "runs are dealt evenly over the waves");
      const int lrow = lane / GPR, lg16 = lane % GPR;
      const unsigned off0 = (unsigned)(lrow * ROWB + ((lg16 ^ (lrow & 7)) << 4));
      const unsigned off1 = (unsigned)(lrow * ROWB + ((lg16 ^ ((RPR + lrow) & 7)) << 4));
#pragma unroll
      for (int k = 0; k < NTL * RUNS / NW; ++k) {
        const int run = w + k * NW;                  // wave-uniform
        const int t = run / RUNS, ri = run % RUNS;
        const E* src = t == 0 ? qg : (t == 1 ? kg : vg);
        const unsigned o = (RPR >= 8 || (ri & 1) == 0) ? off0 : off1;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const unsigned char*>(src) + (unsigned)(ri * 1024) + o,
                                         (__attribute__((address_space(3))) void*)(smem + (t == 0 ? lay.q : t == 1 ? lay.k : lay.v) + ri * 1024),
                                         16, 0, 0);
      }
      const unsigned char* ls = reinterpret_cast<const unsigned char*>(lg);
      if (lam4) {
        for (int ri = w; ri * 1024 < C * L * 4; ri += NW) {
          const unsigned byte = (unsigned)(ri * 1024 + lane * 16);
          if (byte < (unsigned)(C * L * 4))
            __builtin_amdgcn_global_load_lds(ls + byte, (__attribute__((address_space(3))) void*)(smem + lay.lam + ri * 1024), 16, 0, 0);
        }
      } else {
        for (int ri = w; ri * 256 < C * L * 4; ri += NW) {
          const unsigned byte = (unsigned)(ri * 256 + lane * 4);
          if (byte < (unsigned)(C * L * 4))
            __builtin_amdgcn_global_load_lds(ls + byte, (__attribute__((address_space(3))) void*)(smem + lay.lam + ri * 256), 4, 0, 0);
        }
      }
    } else {
      // the partial last chunk: element copies, zeros past the sequence
      const E* srcs[3] = {qg, kg, vg};
      for (int i = tid; i < NTL * C * GPR; i += SH::NT) {
        const int t = i / (C * GPR), rem = i % (C * GPR), r = rem / GPR, g = rem % GPR;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (r < nv) x = *reinterpret_cast<const uint4*>(srcs[t] + (unsigned)(r * D + g * 8));
        *reinterpret_cast<uint4*>(smem + (t == 0 ? lay.q : t == 1 ? lay.k : lay.v) + swz_gran<D>(r, g)) = x;
      }
      for (int i = tid; i < C * L; i += SH::NT) lamS[i] = i < nv * L ? lg[i] : 0.f;
    }
  } else {
#pragma unroll
  for (int p = 0; p < SH::NPF; ++p) {
    const int idx = tid + p * SH::NT;
    const int r = idx / SH::VPR, cv = idx % SH::VPR;   // columns fastest: each row read whole
    qx[p] = kx[p] = vx[p] = make_uint4(0, 0, 0, 0);
    if (idx < SH::NV && r < nv) {
      qx[p] = *reinterpret_cast<const uint4*>(qg + r * D + cv * EPV);
      kx[p] = *reinterpret_cast<const uint4*>(kg + r * D + cv * EPV);
      vx[p] = *reinterpret_cast<const uint4*>(vg + r * D + cv * EPV);
    }
  }
#pragma unroll
  for (int p = 0; p < SH::NLX; ++p) lx[p] = 0.f;
  if (lam4) {
#pragma unroll
    for (int p = 0; p < SH::NPL4; ++p) {
      const int idx = tid + p * SH::NT;
      if (4 * idx < C * L) {
        const float4 f = *reinterpret_cast<const float4*>(lg + 4 * idx);
        lx[4 * p] = f.x; lx[4 * p + 1] = f.y; lx[4 * p + 2] = f.z; lx[4 * p + 3] = f.w;
      }
    }
  } else {
#pragma unroll
    for (int p = 0; p < SH::NPL; ++p) {
      if (p * SH::NT >= C * L) continue;
      const int idx = tid + p * SH::NT;
      if (idx < nv * L) lx[p] = lg[idx];
    }
  }
  }
  // wave 0: the chunk's log gates, KPG consecutive tokens per lane
  constexpr int KPG = C <= 64 ? 1 : 2;
  float lax[KPG];
#pragma unroll
  for (int u = 0; u < KPG; ++u) {
    const int r = KPG * lane + u;
    lax[u] = (w == 0 && r < C && tc + r < T) ? a.log_a[bh * T + tc + r] : 0.f;
  }

  // ---- occupied levels above the chunk, found by every wave from the chunk
  // index alone (lanes 1..LOG2G: chunk levels inside the group; lanes 32..62:
  // group levels); their gates are loaded now and used at contraction time.
  const int64_t gam = c / G, cg0 = gam * G;
  const int ci = (int)(c - cg0);
  bool act = false;
  int64_t off = 0;                                  // node offset from its base (elements)
  int lev = 0, src = 0;
  int64_t eg = 0;
  if (lane >= 1 && lane <= LOG2G) {
    const BucketRef bk = chunk_level_bucket(c, lane, LOG2C, LOG2G);
    if (bk.occupied) {
      const int el = (int)(bk.last - cg0);         // in-group chunk of the node
      act = true;
      off = (bh * nc + bk.last) * D * D;
      src = el + 1;
      lev = bk.level;
    }
  }
  if (lane >= 32 && lane < 63) {
    const BucketRef bk = group_level_bucket(c, lane - 31, LOG2C, LOG2G);
    if (bk.occupied) {
      eg = bk.last;
      act = true;
      off = (bh * ng + eg) * D * D;
      lev = bk.level;
    }
  }
  const unsigned long long lmask = __ballot(act);
  const int n_lev = __popcll(lmask);
  // compact the list: lane li receives the lane that holds entry li (lane 63
  // is never an entry and takes the inactive lanes' writes)
  const int pos = __popcll(lmask & ((1ull << lane) - 1ull));
  const int ent = __builtin_amdgcn_ds_permute((act ? pos : 63) << 2, lane);
  const float gx = (lane < ci) ? a.gch[bh * nc + cg0 + lane] : 0.f;
  const double* gp = a.gprefix + bh * (ng + 1);
  const bool grp = act && lane >= 32;
  const double gpe = grp ? gp[eg + 1] : 0.0;
  const double gpg = grp ? gp[gam] : 0.0;
  // node of entry li: a kernel-argument base plus an offset, so its loads
  // stay global (not flat) loads
  auto node_of = [&](int li) {
    const int el = __builtin_amdgcn_readlane(ent, li);
    const uint64_t o64 = (uint64_t)off;
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)o64, el);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(o64 >> 32), el);
    const int64_t o = (int64_t)(((uint64_t)hi << 32) | lo);
    return (el >= 32 ? reinterpret_cast<const E*>(a.nodes) : reinterpret_cast<const E*>(a.nodes_in)) + o;
  };
  const int cb0 = w * NCB;
  Frag nf[NPRE][KSD][NCB];
  // node fragments as the A operand: row d_v, k-slice of d_k
  auto load_node = [&](int li, Frag (&dst)[KSD][NCB]) {
    const E* nodeT = node_of(li);
#pragma unroll
    for (int s2 = 0; s2 < KSD; ++s2) {
      const int k0 = s2 * KST + lq * KPL;
#pragma unroll
      for (int n = 0; n < NCB; ++n)
        dst[s2][n] = EL::template load_k<D>(nodeT + (16 * (cb0 + n) + lr) * D + k0, k0);
    }
  };
  if (!DIRECT && SH::EARLY && cb0 < DB) {
#pragma unroll
    for (int u = 0; u < NPRE; ++u)
      if (u < n_lev) load_node(u, nf[u]);
  }

  // ---- LDS stores: Q, K and V row-major, lambda rows, gate prefix
  if constexpr (!DIRECT) {
#pragma unroll
  for (int p = 0; p < SH::NPF; ++p) {
    const int idx = tid + p * SH::NT;
    if (idx < SH::NV) {
      const int r = idx / SH::VPR, cv = idx % SH::VPR;
      *reinterpret_cast<uint4*>(Qs + r * lay.ld_row + cv * EPV) = qx[p];
      *reinterpret_cast<uint4*>(Ks + r * lay.ld_row + cv * EPV) = kx[p];
      uint32_t* vrow = reinterpret_cast<uint32_t*>(Vs + r * lay.ld_v + cv * EPV);   // 4-byte aligned rows
      vrow[0] = vx[p].x; vrow[1] = vx[p].y; vrow[2] = vx[p].z; vrow[3] = vx[p].w;
    }
  }
  if (lam4) {
#pragma unroll
    for (int p = 0; p < SH::NPL4; ++p) {
      const int idx = tid + p * SH::NT;
      if (4 * idx < C * L)
        *reinterpret_cast<float4*>(lamS + 4 * idx) = make_float4(lx[4 * p], lx[4 * p + 1], lx[4 * p + 2], lx[4 * p + 3]);
    }
  } else {
#pragma unroll
    for (int p = 0; p < SH::NPL; ++p) {
      if (p * SH::NT >= C * L) continue;
      const int idx = tid + p * SH::NT;
      if (idx < C * L) lamS[idx] = lx[p];
    }
  }
  }
  if (w == 0) {
    // in-chunk prefix of log2(a) and its exp2 (the row gate to the chunk start),
    // the same arithmetic as chunk_gate_scan
    float y[KPG];
    if constexpr (KPG == 1) {
      y[0] = wave_incl_scan(lax[0] * kLog2e);
    } else {
      const float x0 = lax[0] * kLog2e, x1 = lax[1] * kLog2e;
      const float sc = wave_incl_scan(x0 + x1);
      y[0] = sc - x1;
      y[1] = sc;
    }
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
      const int r = KPG * lane + u;
      if (r < C) {
        b2c[r] = y[u];
        e2c[r] = __builtin_amdgcn_exp2f(y[u]);
      }
    }
  }
  // log2 gate of each level from the node's end to the chunk start
  float g2 = 0.f;
  {
    const float incl = wave_incl_scan(gx);
    float S = __shfl_up(incl, 1, 64);
    if (lane == 0) S = 0.f;
    const float pre = __shfl(S, ci, 64);            // group start -> chunk start
    const float Se = __shfl(S, src, 64);
    if (act) g2 = grp ? (float)(gpg - gpe) + pre : pre - Se;
  }
  if constexpr (DIRECT) __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads have landed
  __syncthreads();
  if (DIRECT && SH::EARLY && cb0 < DB) {
#pragma unroll
    for (int u = 0; u < NPRE; ++u)
      if (u < n_lev) load_node(u, nf[u]);
  }

  // ---- phase 1: masked score tiles P[query][key] (bf16 or fp32).  Every
  // wave first forms its score tiles S^T = K Q^T; once all waves are past
  // that point the K tile is dead and P is written over it.
  constexpr int KT = (SH::NST + NW - 1) / NW;      // score tiles per wave (max)
  f32x4 sv[KT];
#pragma unroll
  for (int u = 0; u < KT; ++u) {
    sv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int tau = w + u * NW;
    if (tau >= SH::NST) break;
    int qb = 0;
    while ((qb + 1) * (qb + 2) / 2 <= tau) ++qb;
    const int kb = tau - qb * (qb + 1) / 2;
    const int iq = 16 * qb + lr;
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
      const int k0 = s * KST + lq * KPL;
      Frag kf, qf;
      if constexpr (DIRECT) {
        kf = __builtin_bit_cast(Frag, *reinterpret_cast<const u16x8*>(Kt + swz_gran<D>(16 * kb + lr, k0 / 8)));
        qf = __builtin_bit_cast(Frag, *reinterpret_cast<const u16x8*>(Qt + swz_gran<D>(iq, k0 / 8)));
      } else {
        kf = EL::template load_k<D>(Ks + (16 * kb + lr) * lay.ld_row + k0, k0);
        qf = EL::template load_k<D>(Qs + iq * lay.ld_row + k0, k0);
      }
      sv[u] = EL::mma(kf, qf, sv[u]);
    }
  }
  __syncthreads();                                 // K tile no longer read
#pragma unroll
  for (int u = 0; u < KT; ++u) {
    const int tau = w + u * NW;
    if (tau >= SH::NST) break;
    int qb = 0;
    while ((qb + 1) * (qb + 2) / 2 <= tau) ++qb;
    const int kb = tau - qb * (qb + 1) / 2;
    const int iq = 16 * qb + lr;                   // query of this lane (column of S^T)
    const int j0 = 16 * kb + 4 * lq;               // its four keys j0 .. j0 + 3
    const float b2q = b2c[iq];
    const float4 b2k = *reinterpret_cast<const float4*>(b2c + j0);
    const float bk[4] = {b2k.x, b2k.y, b2k.z, b2k.w};
    float pv[4];
    if (kb < qb) {
      // below the diagonal every pair differs first in the 16-block bits:
      // one level for the whole tile, no causal mask
      const float lam_q = lamS[iq * L + 5 + (31 - __builtin_clz((unsigned)(qb ^ kb)))];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float val = sv[u][i] * __builtin_amdgcn_exp2f(b2q - bk[i]) * lam_q;
        pv[i] = (FULL || iq < nv) ? val : 0.f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // computed for every key and then masked: the level stays within
        // 0..log2 C and the gate exponent past the diagonal is discarded
        const int j = j0 + i;
        const int lv = fenwick_level_local((unsigned)iq, (unsigned)j);
        const float val = sv[u][i] * __builtin_amdgcn_exp2f(b2q - bk[i]) * lamS[iq * L + lv];
        pv[i] = (j <= iq && iq < nv) ? val : 0.f;
      }
    }
    E* prow = Ps + iq * lay.ld_p + j0;
    if constexpr (BF16) {
      *reinterpret_cast<u16x4*>(prow) =
          u16x4{f32_to_bf16(pv[0]), f32_to_bf16(pv[1]), f32_to_bf16(pv[2]), f32_to_bf16(pv[3])};
    } else {
      *reinterpret_cast<float4*>(prow) = make_float4(pv[0], pv[1], pv[2], pv[3]);
    }
  }
  __syncthreads();

  // ---- phase 2: this wave's output columns for all query rows, transposed:
  // acc[rb][n][i] = O[16 rb + lr][16 (cb0 + n) + 4 lq + i]
  if (cb0 >= DB) return;
  if (!SH::EARLY) {
#pragma unroll
    for (int u = 0; u < NPRE; ++u)
      if (u < n_lev) load_node(u, nf[u]);
  }
  f32x4 acc[QB][NCB];
#pragma unroll
  for (int rb = 0; rb < QB; ++rb)
#pragma unroll
    for (int n = 0; n < NCB; ++n) acc[rb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (!VL) {
  // V^T fragments (row d_v, a k-slice of keys) gathered from row-major V
  Frag vf[SH::KSC][NCB];
#pragma unroll
  for (int s = 0; s < SH::KSC; ++s) {
    const int k0 = s * KST + lq * KPL;
#pragma unroll
    for (int n = 0; n < NCB; ++n) {
      const int dv = 16 * (cb0 + n) + lr;
      if constexpr (DIRECT) {
        // C >= 32 here: every k-slice lies inside the chunk
        vf[s][n] = swz_tr_frag<D>(Vt, s * KST, 16 * (cb0 + n), lane);
      } else if constexpr (BF16) {
        u16x8 f = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (C >= KST || k0 < C) {
          const unsigned short* vcol = reinterpret_cast<const unsigned short*>(Vs) + dv;
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = vcol[(k0 + e) * lay.ld_v];
        }
        vf[s][n] = __builtin_bit_cast(Frag, f);
      } else {
        vf[s][n] = Vs[k0 * lay.ld_v + dv];
      }
    }
  }
  // O^T = V^T P^T over keys 0 .. 16 rb + 15 of each row block
#pragma unroll
  for (int rb = 0; rb < QB; ++rb) {
#pragma unroll
    for (int s = 0; s < SH::KSC; ++s) {
      if (s * KST > 16 * rb + 15) break;
      const int k0 = s * KST + lq * KPL;
      Frag pb;
      if (k0 / 16 <= rb) pb = EL::load(Ps + (16 * rb + lr) * lay.ld_p + k0);
      else if constexpr (BF16) pb = __builtin_bit_cast(Frag, u16x8{0, 0, 0, 0, 0, 0, 0, 0});
      else pb = 0.f;
#pragma unroll
      for (int n = 0; n < NCB; ++n) acc[rb][n] = EL::mma(vf[s][n], pb, acc[rb][n]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  }

  // ---- occupied levels above the chunk: O += diag(lambda * gate) Q node^T,
  // two levels per pass so that each Q fragment is read once for both (the
  // second level's terms are still added after the first's).  The row gate
  // exp2(b) and the bucket gate exp2(gate2) are both <= 1.
  auto level_of = [&](int li, float& f, int& lv) {
    const int el = __builtin_amdgcn_readlane(ent, li);
    f = __builtin_amdgcn_exp2f(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g2), el)));
    lv = __builtin_amdgcn_readlane(lev, el);
  };
  auto contract2 = [&](int li, const Frag (&nf0)[KSD][NCB], bool two, const Frag (&nf1)[KSD][NCB]) {
    float f0, f1 = 0.f;
    int lv0, lv1 = 0;
    level_of(li, f0, lv0);
    if (two) level_of(li + 1, f1, lv1);
#pragma unroll
    for (int rb = 0; rb < QB; ++rb) {
      f32x4 t0[NCB], t1[NCB];
#pragma unroll
      for (int n = 0; n < NCB; ++n) t0[n] = t1[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < KSD; ++s2) {
        const int k0 = s2 * KST + lq * KPL;
        Frag qf;
        if constexpr (DIRECT) qf = __builtin_bit_cast(Frag, *reinterpret_cast<const u16x8*>(Qt + swz_gran<D>(16 * rb + lr, k0 / 8)));
        else qf = EL::template load_k<D>(Qs + (16 * rb + lr) * lay.ld_row + k0, k0);
#pragma unroll
        for (int n = 0; n < NCB; ++n) {
          t0[n] = EL::mma(nf0[s2][n], qf, t0[n]);
          if (two) t1[n] = EL::mma(nf1[s2][n], qf, t1[n]);
        }
      }
      const int r = 16 * rb + lr;                   // this lane's query row
      const float e = e2c[r];
      const float w0 = lamS[r * L + lv0] * e * f0;
#pragma unroll
      for (int n = 0; n < NCB; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rb][n][i] += w0 * t0[n][i];
      if (two) {
        const float w1 = lamS[r * L + lv1] * e * f1;
#pragma unroll
        for (int n = 0; n < NCB; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][n][i] += w1 * t1[n][i];
      }
      // keep the next row block's Q fragments from being hoisted: live ranges
      // stay one row block long
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // ring of NPRE (even) fragment buffers: level li uses buffer li % NPRE and,
  // once multiplied, the buffer takes level li + NPRE
  static_assert(NPRE % 2 == 0, "levels are contracted in pairs");
  for (int base = 0; base < n_lev; base += NPRE) {
#pragma unroll
    for (int u = 0; u < NPRE; u += 2) {
      const int li = base + u;
      if (li >= n_lev) break;
      const bool two = li + 1 < n_lev;
      contract2(li, nf[u], two, nf[u + 1]);
      if (li + NPRE < n_lev) load_node(li + NPRE, nf[u]);
      if (li + 1 + NPRE < n_lev) load_node(li + 1 + NPRE, nf[u + 1]);
    }
  }

  if constexpr (VL) {
    // ---- V into the Q tile, then O^T += V^T P^T
    __syncthreads();                               // every wave is past its Q reads
    if (FULL) {
      constexpr int ROWB = 2 * D, GPR = ROWB / 16, RPR = 1024 / ROWB, RUNS = C * ROWB / 1024;
      static_assert(RUNS % NW == 0, "runs are dealt evenly over the waves");
      const int lrow = lane / GPR, lg16 = lane % GPR;
      const unsigned off0 = (unsigned)(lrow * ROWB + ((lg16 ^ (lrow & 7)) << 4));
      const unsigned off1 = (unsigned)(lrow * ROWB + ((lg16 ^ ((RPR + lrow) & 7)) << 4));
#pragma unroll
      for (int k = 0; k < RUNS / NW; ++k) {
        const int ri = w + k * NW;                 // wave-uniform
        const unsigned o = (RPR >= 8 || (ri & 1) == 0) ? off0 : off1;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const unsigned char*>(vg) + (unsigned)(ri * 1024) + o,
                                         (__attribute__((address_space(3))) void*)(smem + lay.v + ri * 1024),
                                         16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0);               // this wave's direct loads have landed
    } else {
      constexpr int GPR = 2 * D / 16;
      for (int i = tid; i < C * GPR; i += SH::NT) {
        const int r = i / GPR, g = i % GPR;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (r < nv) x = *reinterpret_cast<const uint4*>(vg + (unsigned)(r * D + g * 8));
        *reinterpret_cast<uint4*>(smem + lay.v + swz_gran<D>(r, g)) = x;
      }
    }
    __syncthreads();
    // V^T fragments (row d_v, a k-slice of keys) gathered from row-major V
    Frag vf[SH::KSC][NCB];
  #pragma unroll
    for (int s = 0; s < SH::KSC; ++s) {
      const int k0 = s * KST + lq * KPL;
  #pragma unroll
      for (int n = 0; n < NCB; ++n) {
        const int dv = 16 * (cb0 + n) + lr;
        if constexpr (DIRECT) {
          // C >= 32 here: every k-slice lies inside the chunk
          vf[s][n] = swz_tr_frag<D>(Vt, s * KST, 16 * (cb0 + n), lane);
        } else if constexpr (BF16) {
          u16x8 f = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
          if (C >= KST || k0 < C) {
            const unsigned short* vcol = reinterpret_cast<const unsigned short*>(Vs) + dv;
  #pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = vcol[(k0 + e) * lay.ld_v];
          }
          vf[s][n] = __builtin_bit_cast(Frag, f);
        } else {
          vf[s][n] = Vs[k0 * lay.ld_v + dv];
        }
      }
    }
    // O^T = V^T P^T over keys 0 .. 16 rb + 15 of each row block
  #pragma unroll
    for (int rb = 0; rb < QB; ++rb) {
  #pragma unroll
      for (int s = 0; s < SH::KSC; ++s) {
        if (s * KST > 16 * rb + 15) break;
        const int k0 = s * KST + lq * KPL;
        Frag pb;
        if (k0 / 16 <= rb) pb = EL::load(Ps + (16 * rb + lr) * lay.ld_p + k0);
        else if constexpr (BF16) pb = __builtin_bit_cast(Frag, u16x8{0, 0, 0, 0, 0, 0, 0, 0});
        else pb = 0.f;
  #pragma unroll
        for (int n = 0; n < NCB; ++n) acc[rb][n] = EL::mma(vf[s][n], pb, acc[rb][n]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- store.  Direct-load tiles whose column blocks the waves cover
  // exactly (every wave owns output columns): the output tile is staged in the
  // dead Q (or late V) tile, swizzled like it, and written as whole rows, 16
  // bytes per lane (1 KB of rows per wave instruction); else four consecutive
  // output columns of one row per lane and block.
  constexpr bool STAGE_OUT = DIRECT && NW * NCB == DB;
  if constexpr (STAGE_OUT) {
    unsigned char* Ot = smem + lay.q;
    __syncthreads();                               // every wave is past its Q and V reads
#pragma unroll
    for (int rb = 0; rb < QB; ++rb) {
      const int r = 16 * rb + lr;
#pragma unroll
      for (int n = 0; n < NCB; ++n) {
        const int c = 16 * (cb0 + n) + 4 * lq;
        *reinterpret_cast<u16x4*>(Ot + swz_gran<D>(r, c / 8) + (c % 8) * 2) =
            u16x4{f32_to_bf16(acc[rb][n][0]), f32_to_bf16(acc[rb][n][1]), f32_to_bf16(acc[rb][n][2]),
                  f32_to_bf16(acc[rb][n][3])};
      }
    }
    __syncthreads();
    constexpr int GPR = 2 * D / 16;
    for (int idx = tid; idx < C * GPR; idx += SH::NT) {
      const int r = idx / GPR, g = idx % GPR;
      if (r < nv) *reinterpret_cast<uint4*>(og + (int64_t)r * D + g * 8) = *reinterpret_cast<const uint4*>(Ot + swz_gran<D>(r, g));
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < QB; ++rb) {
      const int r = 16 * rb + lr;
      if (r < nv) {
#pragma unroll
        for (int n = 0; n < NCB; ++n) {
          E* o = og + (int64_t)r * D + 16 * (cb0 + n) + 4 * lq;
          if constexpr (BF16) {
            *reinterpret_cast<u16x4*>(o) = u16x4{f32_to_bf16(acc[rb][n][0]), f32_to_bf16(acc[rb][n][1]),
                                                 f32_to_bf16(acc[rb][n][2]), f32_to_bf16(acc[rb][n][3])};
          } else {
            *reinterpret_cast<float4*>(o) = make_float4(acc[rb][n][0], acc[rb][n][1], acc[rb][n][2], acc[rb][n][3]);
          }
        }
      }
    }
  }
}

// Work item of a block.  Blocks are dealt to the 8 XCDs round-robin (block b
// runs on XCD b % 8, each XCD with its own L2); renumbered so that every XCD
// walks one contiguous run of (b,h, chunk) items, the chunks that share the
// upper level nodes meet in one L2.
__device__ __forceinline__ int64_t xcd_item(int64_t b, int64_t n) {
  constexpr int X = 8;
  const int64_t q = n / X, r = n % X, x = b % X, i = b / X;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// The kernel is bound by memory latency, so where the register budget of 4
// waves per SIMD (128) costs no spills -- bf16 tiles up to 64 x 64, those
// that load the first nodes early -- the compiler is held to it.
template <bool BF16, int C, int D>
constexpr int output_min_waves() { return ChunkShape<BF16, C, D>::EARLY ? (output_direct(C, D, BF16 ? 2 : 4) ? 5 : 4) : 1; }

template <bool BF16, int C, int D>
__global__ __launch_bounds__(64 * output_waves(C)) __attribute__((amdgpu_waves_per_eu(output_min_waves<BF16, C, D>(), 8)))
void fwd_chunk_output(FwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t item = xcd_item(blockIdx.x, gridDim.x);
  const int64_t c = (uint32_t)item % (uint32_t)a.n_chunks;
  if ((c + 1) * C <= a.T) chunk_output_body<BF16, C, D, true>(a, smem, item);
  else chunk_output_body<BF16, C, D, false>(a, smem, item);
}

// The late-V output kernel (bfloat16, C = d = 64 or 128).  At C = 128 two
// workgroups of eight waves share a CU: the register budget of four waves per
// SIMD.  At C = 64 the LDS admits seven workgroups of four waves, so the
// registers decide: the budget of six waves per SIMD (80 VGPRs).
constexpr int output_vlate_min_waves(int C) { return C == 64 ? 6 : 4; }
template <bool BF16, int C, int D>
__global__ __launch_bounds__(64 * output_waves(C)) __attribute__((amdgpu_waves_per_eu(output_vlate_min_waves(C), 8)))
void fwd_chunk_output_vlate(FwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t item = xcd_item(blockIdx.x, gridDim.x);
  const int64_t c = (uint32_t)item % (uint32_t)a.n_chunks;
  if ((c + 1) * C <= a.T) chunk_output_body<BF16, C, D, true, true>(a, smem, item);
  else chunk_output_body<BF16, C, D, false, true>(a, smem, item);
}

// ---------------------------------------------------------------------------
// Host-side launch of the stages for one (dtype, C, D) instantiation.
template <bool BF16, int C, int D>
int launch_fwd_impl(const FwdPlan& p, FwdArgs a, hipStream_t s, hipEvent_t const* ev) {
  using E = typename Elem<BF16>::T;
  constexpr int G = state_group(D);
  if (p.G != G) return kEHIP;
  int stage = 0;
  bool ok = true;
  auto mark = [&]() {
    if (ev) ok = ok && hipEventRecord(ev[stage], s) == hipSuccess;
    ++stage;
  };
  const bool final_state = a.st_slots != nullptr;
  if (p.n_chunks > 1 || (final_state && p.has_chunk_nodes())) {
    constexpr int lds_s = state_lds(C, D, sizeof(E), G).total;
    ok = ok && hipFuncSetAttribute((const void*)fwd_chunk_states<BF16, C, D>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds_s) == hipSuccess;
    if (!ok) return kEHIP;
    mark();
    hipLaunchKernelGGL((fwd_chunk_states<BF16, C, D>), dim3((unsigned)(p.n_groups * p.BH)),
                       dim3(StateShape<BF16, C, D>::NT), lds_s, s, a);
    ok = ok && hipGetLastError() == hipSuccess;
  }
  if (p.n_groups > 1 || (final_state && p.has_group_nodes())) {
    mark();
    const dim3 grid((unsigned)(group_tree_blocks(D) * p.BH));
    const int levels = bit_length(p.n_groups);        // carry levels the walk can reach
    if (levels <= 6)
      hipLaunchKernelGGL((fwd_group_tree<BF16, 6>), grid, dim3(kTreeThreads), 0, s, a, D);
    else if (levels <= 8)
      hipLaunchKernelGGL((fwd_group_tree<BF16, 8>), grid, dim3(kTreeThreads), 0, s, a, D);
    else if (levels <= 16)
      hipLaunchKernelGGL((fwd_group_tree<BF16, 16>), grid, dim3(kTreeThreads), 0, s, a, D);
    else
      hipLaunchKernelGGL((fwd_group_tree<BF16, 32>), grid, dim3(kTreeThreads), 0, s, a, D);
    ok = ok && hipGetLastError() == hipSuccess;
  }
  bool launched = false;
  if constexpr (output_vlate_shape(C, D, sizeof(E))) {
    if (p.lds_out_vlate > 0) {
      ok = ok && hipFuncSetAttribute((const void*)fwd_chunk_output_vlate<BF16, C, D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_out_vlate) == hipSuccess;
      if (!ok) return kEHIP;
      mark();
      hipLaunchKernelGGL((fwd_chunk_output_vlate<BF16, C, D>), dim3((unsigned)(p.n_chunks * p.BH)),
                         dim3(ChunkShape<BF16, C, D>::NT), p.lds_out_vlate, s, a);
      ok = ok && hipGetLastError() == hipSuccess;
      launched = true;
    }
  }
  if (!launched) {
    ok = ok && hipFuncSetAttribute((const void*)fwd_chunk_output<BF16, C, D>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_out) == hipSuccess;
    if (!ok) return kEHIP;
    mark();
    hipLaunchKernelGGL((fwd_chunk_output<BF16, C, D>), dim3((unsigned)(p.n_chunks * p.BH)),
                       dim3(ChunkShape<BF16, C, D>::NT), p.lds_out, s, a);
    ok = ok && hipGetLastError() == hipSuccess;
  }
  if (final_state) {
    hipLaunchKernelGGL((fwd_final_state<BF16, C, D>), dim3((unsigned)p.BH), dim3(256), 0, s, a);
    ok = ok && hipGetLastError() == hipSuccess;
  }
  if (ev) ok = ok && hipEventRecord(ev[stage], s) == hipSuccess;
  return ok ? kOK : kEHIP;
}

template <bool BF16>
int launch_fwd_dtype(const FwdPlan& p, FwdArgs a, hipStream_t s, hipEvent_t const* ev) {
#define LA_CASE(CC, DD) \
  if (p.C == CC && p.D == DD) return launch_fwd_impl<BF16, CC, DD>(p, a, s, ev);
  LA_CASE(16, 16) LA_CASE(16, 32) LA_CASE(16, 64) LA_CASE(16, 128)
  LA_CASE(32, 16) LA_CASE(32, 32) LA_CASE(32, 64) LA_CASE(32, 128)
  LA_CASE(64, 16) LA_CASE(64, 32) LA_CASE(64, 64) LA_CASE(64, 128)
  LA_CASE(128, 16) LA_CASE(128, 32) LA_CASE(128, 64) LA_CASE(128, 128)
#undef LA_CASE
  return kESHAPE;
}

}  // namespace la
