// Kernels of the Log-Linear Mamba-2 layer around the operator (gfx950):
//
//   gemm_nt          C = A B^T on the matrix cores: the input projection
//                    (u -> z | x | B | C | dt | lam columns) and the output
//                    projection
//   mamba2_prologue  causal depthwise conv + silu of the x | B | C columns,
//                    softplus gates, and the operator's inputs in its own
//                    layout: q = C, k = B (per head of each group),
//                    v = dt x, log_a = dt A, lambda = softplus(. + bias)
//   mamba2_gate_norm y = o + D x (x recomputed from the conv), times silu(z),
//                    normalised by the root mean square over each group of
//                    channels, times the norm weight
//
// The layer is Mamba-2's block with its SSM replaced by the log-linear
// operator ("Log-Linear Attention", Spanish summary, technical section 2,
// "Variantes", item 1: Mamba-2's selective gate with the hierarchical mask);
// the block itself (projections, conv, gates, gated norm) follows Mamba-2's
// published design, since the pages give no layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_device.hpp"
#include "la_layer_plan.hpp"

namespace la {

struct GemmArgs {
  const void* A;   // [M][lda], rows 16-byte aligned
  const void* B;   // [N][ldb]
  void* C;         // [M][ldc]
  int M, N, K, lda, ldb, ldc;   // K a multiple of two K-slices; ldc a multiple of 4
  int tiles_n, tiles;           // column tiles, all tiles
};

constexpr int kGemmTM = kGemmTile;                               // rows of a workgroup tile
constexpr int kGemmTN = kGemmTile;                               // columns of a workgroup tile
constexpr int kGemmStageBytes = (kGemmTM + kGemmTN) * kGemmKBytes; // A and B slices of one stage
// LDS of a workgroup: the double buffer, which the epilogue reuses to stage
// one 32-row block of every wave's results (rows padded by 8 bytes; fp32
// blocks are larger than the buffers)
constexpr int kGemmStage32 = 4 * 32 * (128 * 4 + 8);
constexpr int kGemmLds = 2 * kGemmStageBytes > kGemmStage32 ? 2 * kGemmStageBytes : kGemmStage32;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// C[m][n] = sum_k A[m][k] B[n][k], fp32 accumulation, rounded to the element
// type.  A workgroup of four waves computes a 256 x 256 tile, each wave a
// 128 x 128 quarter as 4 x 4 tiles of 32 x 32 on the matrix cores
// (v_mfma_f32_32x32x16_bf16; fp32: v_mfma_f32_32x32x2f32, four k-steps per
// 16-byte granule, element c of every lane's granule feeding step c), its 256
// accumulators per lane in the accumulation registers, one wave per SIMD.
// The large wave tile keeps the LDS traffic per multiply-add low enough for
// the matrix cores: 512 bytes of fragments per k for 16384 MACs (a 64 x 64
// tile needs twice that per MAC, which the LDS cannot feed).  K-slices
// (kGemmKBytes bytes of every row of the A and B tiles) are double-buffered in
// LDS and run two slices ahead in registers: slice kt + 2 is loaded while
// slice kt is multiplied and slice kt + 1, loaded one step earlier, waits to be
// written to the free buffer.  A slice row's four 16-byte granules are stored
// XOR-swizzled (granule g of row r at slot g ^ ((r >> 2) & 3)), so the eight
// rows one LDS cycle of a fragment read serves fall in distinct banks.  Rows
// past M or N are clamped to the last row for loading and never stored.
template <bool BF16>
__global__ __launch_bounds__(256, 1) void gemm_nt(GemmArgs g) {
  using E = Elem<BF16>;
  using T = typename E::T;
  constexpr int ES = sizeof(T);
  constexpr int TM = kGemmTM, TN = kGemmTN, ROWB = kGemmKBytes, GPR = ROWB / 16;
  static_assert(GPR == 4 && TM == 256 && TN == 256, "256 x 256 tiles of four-granule slice rows");
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // XCD-major tile order: consecutive workgroups are dealt round-robin over the
  // 8 XCDs, so renumber them so that one XCD sweeps the column tiles of a row
  // tile while that row tile sits in its L2
  const int nblk = gridDim.x, per = nblk / 8;
  int blk = blockIdx.x;
  if (blk < per * 8) blk = (blk % 8) * per + blk / 8;
  const int m0 = (blk / g.tiles_n) * TM, n0 = (blk % g.tiles_n) * TN;

  // loads: thread t moves granule t % 4 of rows t / 4 + 64 j (j < 4) of both
  // tiles; four consecutive threads cover one 64-byte slice row
  const int lrow = tid >> 2, lgr = tid & 3;
  const unsigned char* pa[4];
  const unsigned char* pb[4];
  int sw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = lrow + 64 * j;
    pa[j] = static_cast<const unsigned char*>(g.A) + (size_t)min(m0 + r, g.M - 1) * g.lda * ES + lgr * 16;
    pb[j] = static_cast<const unsigned char*>(g.B) + (size_t)min(n0 + r, g.N - 1) * g.ldb * ES + lgr * 16;
    sw[j] = r * ROWB + ((lgr ^ ((r >> 2) & 3)) << 4);
  }
  const int nk = g.K * ES / ROWB;   // even
  // four register sets of eight granules, named (an array here would live in
  // scratch memory: it is promoted to registers before the loops unroll)
  uint4 a0, a1, a2, a3, a4, a5, a6, a7, b0, b1, b2, b3, b4, b5, b6, b7;
  uint4 c0, c1, c2, c3, c4, c5, c6, c7, d0, d1, d2, d3, d4, d5, d6, d7;
#define LA_GEMM_GLOAD(x0, x1, x2, x3, y0, y1, y2, y3, kt)                  \
  do {                                                                      \
    const size_t ko = (size_t)min(kt, nk - 1) * ROWB;                       \
    x0 = *reinterpret_cast<const uint4*>(pa[0] + ko);                       \
    x1 = *reinterpret_cast<const uint4*>(pa[1] + ko);                       \
    x2 = *reinterpret_cast<const uint4*>(pa[2] + ko);                       \
    x3 = *reinterpret_cast<const uint4*>(pa[3] + ko);                       \
    y0 = *reinterpret_cast<const uint4*>(pb[0] + ko);                       \
    y1 = *reinterpret_cast<const uint4*>(pb[1] + ko);                       \
    y2 = *reinterpret_cast<const uint4*>(pb[2] + ko);                       \
    y3 = *reinterpret_cast<const uint4*>(pb[3] + ko);                       \
  } while (0)
#define LA_GEMM_SWRITE(x0, x1, x2, x3, y0, y1, y2, y3, buf)                 \
  do {                                                                      \
    unsigned char* base = smem + (buf) * kGemmStageBytes;                   \
    *reinterpret_cast<uint4*>(base + sw[0]) = x0;                           \
    *reinterpret_cast<uint4*>(base + sw[1]) = x1;                           \
    *reinterpret_cast<uint4*>(base + sw[2]) = x2;                           \
    *reinterpret_cast<uint4*>(base + sw[3]) = x3;                           \
    *reinterpret_cast<uint4*>(base + TM * ROWB + sw[0]) = y0;               \
    *reinterpret_cast<uint4*>(base + TM * ROWB + sw[1]) = y1;               \
    *reinterpret_cast<uint4*>(base + TM * ROWB + sw[2]) = y2;               \
    *reinterpret_cast<uint4*>(base + TM * ROWB + sw[3]) = y3;               \
  } while (0)

  const int wm = w >> 1, wn = w & 1, fr = lane & 31, fq = lane >> 5;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // the products of the slice in LDS buffer `buf`; B is the first operand, so
  // lane l then holds, for element e, C row 32 i + l % 32 at column
  // 32 j + 8 (e / 4) + 4 (l / 32) + e % 4
#define LA_GEMM_FRAGS(af, bf, As, Bs, ks)                                                                  \
  do {                                                                                                     \
    const int slot = ((2 * (ks) + fq) ^ ((fr >> 2) & 3)) << 4;                                             \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                          \
      af[i] = *reinterpret_cast<const uint4*>(As + (wm * 128 + 32 * i + fr) * ROWB + slot);                \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                          \
      bf[j] = *reinterpret_cast<const uint4*>(Bs + (wn * 128 + 32 * j + fr) * ROWB + slot);                \
  } while (0)
#define LA_GEMM_STEP(af, bf)                                                                               \
  do {                                                                                                     \
    if constexpr (BF16) {                                                                                  \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                        \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                      \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bf[j]),           \
                                                              __builtin_bit_cast(bf16x8, af[i]),           \
                                                              acc[i][j], 0, 0, 0);                         \
    } else {                                                                                               \
      _Pragma("unroll") for (int c = 0; c < 4; ++c)                                                        \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                      \
          _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                    \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, (&bf[j].x)[c]),     \
                                                             __builtin_bit_cast(float, (&af[i].x)[c]),     \
                                                             acc[i][j], 0, 0, 0);                          \
    }                                                                                                      \
  } while (0)
  // the two k-steps of the slice in LDS buffer `buf`: the second step's
  // fragments are read while the first step's products run
#define LA_GEMM_MMA(buf)                                                                                   \
  do {                                                                                                     \
    const unsigned char* As = smem + (buf) * kGemmStageBytes;                                              \
    const unsigned char* Bs = As + TM * ROWB;                                                              \
    uint4 af0[4], bf0[4], af1[4], bf1[4];                                                                  \
    LA_GEMM_FRAGS(af0, bf0, As, Bs, 0);                                                                    \
    LA_GEMM_FRAGS(af1, bf1, As, Bs, 1);                                                                    \
    LA_GEMM_STEP(af0, bf0);                                                                                \
    LA_GEMM_STEP(af1, bf1);                                                                                \
  } while (0)

  // Slice s is in register set s % 4 from four slices before it is
  // multiplied; it is written to LDS buffer s % 2 at the end of step s - 1,
  // multiplied in step s, and its register set then takes slice s + 4.  Every
  // buffer written was last read before the preceding barrier.  Loads past the
  // last slice fetch the last one again; their products are skipped.
#define LA_GEMM_HALF(S, X, Y)                                                                  \
  do {                                                                                         \
    LA_GEMM_GLOAD(X##0, X##1, X##2, X##3, X##4, X##5, X##6, X##7, (S) + 4);                    \
    __builtin_amdgcn_sched_barrier(0);   /* keep the loads ahead of the products */            \
    if ((S) < nk) LA_GEMM_MMA((S) & 1);                                                        \
    LA_GEMM_SWRITE(Y##0, Y##1, Y##2, Y##3, Y##4, Y##5, Y##6, Y##7, ((S) + 1) & 1);             \
    __syncthreads();                                                                           \
  } while (0)
  LA_GEMM_GLOAD(a0, a1, a2, a3, a4, a5, a6, a7, 0);
  LA_GEMM_GLOAD(b0, b1, b2, b3, b4, b5, b6, b7, 1);
  LA_GEMM_GLOAD(c0, c1, c2, c3, c4, c5, c6, c7, 2);
  LA_GEMM_GLOAD(d0, d1, d2, d3, d4, d5, d6, d7, 3);
  LA_GEMM_SWRITE(a0, a1, a2, a3, a4, a5, a6, a7, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 4) {
    LA_GEMM_HALF(kt, a, b);
    LA_GEMM_HALF(kt + 1, b, c);
    LA_GEMM_HALF(kt + 2, c, d);
    LA_GEMM_HALF(kt + 3, d, a);
  }
#undef LA_GEMM_HALF
#undef LA_GEMM_GLOAD
#undef LA_GEMM_SWRITE
#undef LA_GEMM_MMA
#undef LA_GEMM_FRAGS
#undef LA_GEMM_STEP

  // store through LDS, so that every global store is a whole 256-byte row
  // segment (a lane's own results are four columns of one row: stored
  // directly, a row would take many partial-line writes): per block i of 32
  // rows, each wave writes its 32 x 128 results to LDS (rows padded to an
  // 8-byte offset mod 256, so the 32 rows of one store instruction hit
  // distinct banks), then reads 16-byte pieces back along the rows
  constexpr int SROW = 128 * ES + 8;                 // padded LDS row of a wave's block
  unsigned char* st = smem + w * 32 * SROW;
  const int lr = lane >> 4, lc = lane & 15;          // read-back: 4 rows x 16 pieces per instruction
  constexpr int PPR = 128 * ES / 16;                 // 16-byte pieces per row of the block
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int c = 32 * j + 8 * e4 + 4 * fq;
        const float v0 = acc[i][j][4 * e4], v1 = acc[i][j][4 * e4 + 1], v2 = acc[i][j][4 * e4 + 2],
                    v3 = acc[i][j][4 * e4 + 3];
        if constexpr (BF16) {
          const unsigned lo = (unsigned)E::from_f32(v0) | ((unsigned)E::from_f32(v1) << 16);
          const unsigned hi = (unsigned)E::from_f32(v2) | ((unsigned)E::from_f32(v3) << 16);
          *reinterpret_cast<uint2*>(st + fr * SROW + c * ES) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<float2*>(st + fr * SROW + c * ES) = make_float2(v0, v1);
          *reinterpret_cast<float2*>(st + fr * SROW + c * ES + 8) = make_float2(v2, v3);
        }
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's LDS writes done (lgkmcnt 0)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int rr = 0; rr < 32; rr += 4) {
      // lane 16 r' + p reads piece p (+ 16 per round) of row rr + r'
      const int row = rr + lr;
      const int m = m0 + wm * 128 + 32 * i + row;
#pragma unroll
      for (int p0 = 0; p0 < PPR; p0 += 16) {
        const int p = p0 + lc;
        const int n = n0 + wn * 128 + p * (16 / ES);
        const uint4 v = *reinterpret_cast<const uint4*>(st + row * SROW + p * 16);
        if (m < g.M) {
          T* dst = static_cast<T*>(g.C) + (size_t)m * g.ldc + n;
          if (n + 16 / ES <= g.N) {
            *reinterpret_cast<uint4*>(dst) = v;
          } else {
            const T* vv = reinterpret_cast<const T*>(&v);
#pragma unroll
            for (int e = 0; e < 16 / ES; ++e)
              if (n + e < g.N) dst[e] = vv[e];
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // reads done before the next block overwrites
    __builtin_amdgcn_wave_barrier();
  }
}

struct LayerArgs {
  const void* zx;        // [B T][ld_zx] input projection, columns z | x | B | C | dt | lam
  const void* conv_w;    // [conv_dim][K]
  const void* conv_b;    // [conv_dim]
  const float* dt_bias;  // [H]
  const float* A_log;    // [H]
  const float* D;        // [H]
  const float* lam_bias; // [H][L]
  const void* norm_w;    // [d_inner]
  float* taps;           // [conv_dim][kMaxConvTaps + 1] fp32: taps right-aligned, then the bias
  void* q;               // [B][H][T][N]
  void* k;               // [B][H][T][N]
  void* v;               // [B][H][T][P]
  float* log_a;          // [B][H][T]
  float* lam;            // [B][H][T][L]
  const void* o;         // [B][H][T][P] operator output
  void* y;               // [B T][d_inner] normalised gated output
  int64_t T;
  int H, P, N, G, K, L, d_inner, conv_dim, ld_zx;
  int col_x, col_b, col_c, col_dt, col_lam;
  int norm_slots;
  float eps;
};

__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }
// silu with the hardware exponential and reciprocal (a few ulp): x / (1 + e^-x)
__device__ __forceinline__ float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

template <bool BF16, int VEC>
__device__ __forceinline__ void load_vec(const typename Elem<BF16>::T* p, float (&x)[VEC]) {
  if constexpr (BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const unsigned w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __builtin_bit_cast(float, w4[e] << 16);
      x[2 * e + 1] = __builtin_bit_cast(float, w4[e] & 0xffff0000u);
    }
  } else {
    const float4 u = *reinterpret_cast<const float4*>(p);
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
  }
}

template <bool BF16, int VEC>
__device__ __forceinline__ void unpack(const uint4 u, float (&x)[VEC]) {
  if constexpr (BF16) {
    const unsigned w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __builtin_bit_cast(float, w4[e] << 16);
      x[2 * e + 1] = __builtin_bit_cast(float, w4[e] & 0xffff0000u);
    }
  } else {
    x[0] = __builtin_bit_cast(float, u.x); x[1] = __builtin_bit_cast(float, u.y);
    x[2] = __builtin_bit_cast(float, u.z); x[3] = __builtin_bit_cast(float, u.w);
  }
}

template <bool BF16, int VEC>
__device__ __forceinline__ void store_vec(typename Elem<BF16>::T* p, const float (&x)[VEC]) {
  if constexpr (BF16) {
    unsigned w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w4[e] = (unsigned)f32_to_bf16(x[2 * e]) | ((unsigned)f32_to_bf16(x[2 * e + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
}

// The conv taps as fp32, right-aligned in kMaxConvTaps slots (a K-tap conv
// runs as a kMaxConvTaps-tap one whose leading taps are zero), followed by the
// bias: one 20-byte row per channel, read by the conv kernels as a float4 and
// a float.
template <bool BF16>
__global__ __launch_bounds__(256) void mamba2_taps(LayerArgs a) {
  using E = Elem<BF16>;
  using T = typename E::T;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= a.conv_dim) return;
  const T* cw = static_cast<const T*>(a.conv_w) + (size_t)c * a.K;
  const int pad = kMaxConvTaps - a.K;
  float* row = a.taps + (size_t)c * (kMaxConvTaps + 1);
  for (int j = 0; j < kMaxConvTaps; ++j) row[j] = j >= pad ? E::to_f32(cw[j - pad]) : 0.f;
  row[kMaxConvTaps] = E::to_f32(static_cast<const T*>(a.conv_b)[c]);
}

template <int VEC>
__device__ __forceinline__ void load_taps(const float* taps, int c0, float (&w)[VEC][kMaxConvTaps], float (&bias)[VEC]) {
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const float* r = taps + (size_t)(c0 + e) * (kMaxConvTaps + 1);
#pragma unroll
    for (int j = 0; j < kMaxConvTaps; ++j) w[e][j] = r[j];
    bias[e] = r[kMaxConvTaps];
  }
}

constexpr int kSlabGranules = 16;   // conv channels per prologue workgroup, in 16-byte granules
constexpr int kHalo = kMaxConvTaps - 1;
constexpr int kSlabHeads = 16;      // x heads one slab can touch: 128 channels over heads of P >= 16

// Grid (token tiles of kPrologueTokens, sequences, conv slabs + 1).  A conv
// slab stages kHalo + 64 rows of its 16 granules of conv input in LDS (rows
// before the first token are zero), then thread (granule g, block tb) forms
// the conv + silu of tokens 4 tb .. 4 tb + 3 and stores them where the
// operator reads them: v = dt x for x channels, q / k of the group (read by
// all of its heads) for C / B channels.  The last slab writes the gates: lambda of head
// h as one contiguous [tokens, L] block, and log_a.
template <bool BF16>
__global__ __launch_bounds__(256) void mamba2_prologue(LayerArgs a, int n_slabs) {
  using E = Elem<BF16>;
  using T = typename E::T;
  constexpr int VEC = 16 / sizeof(T), TOK = kPrologueTokens, SG = kSlabGranules;
  __shared__ uint4 xs[TOK + kHalo][SG];
  __shared__ float dtS[TOK][kSlabHeads];
  const int b = blockIdx.y, slab = blockIdx.z, tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * TOK;
  const int nt = (int)min((int64_t)TOK, a.T - t0);
  const T* zx = static_cast<const T*>(a.zx) + (size_t)b * a.T * a.ld_zx;
  const int H = a.H;
  const size_t bh0 = (size_t)b * H;

  if (slab == n_slabs) {
    // gates: lambda blocks (coalesced stores, short row gathers), then log_a
    const int per_head = nt * a.L;
    for (int j = tid; j < H * per_head; j += 256) {
      const int h = j / per_head, r = j % per_head, i = r / a.L, l = r % a.L;
      const float raw = E::to_f32(zx[(t0 + i) * a.ld_zx + a.col_lam + h * a.L + l]);
      a.lam[((bh0 + h) * a.T + t0) * a.L + r] = softplus_f(raw + a.lam_bias[h * a.L + l]);
    }
    for (int j = tid; j < H * nt; j += 256) {
      const int h = j / nt, i = j % nt;
      const float raw = E::to_f32(zx[(t0 + i) * a.ld_zx + a.col_dt + h]);
      a.log_a[(bh0 + h) * a.T + t0 + i] = -expf(a.A_log[h]) * softplus_f(raw + a.dt_bias[h]);
    }
    return;
  }

  const int CG = a.conv_dim / VEC, g0 = slab * SG, ng = min(SG, CG - g0);
  for (int i = tid; i < (nt + kHalo) * SG; i += 256) {
    const int r = i / SG, g = i % SG;
    const int64_t t = t0 - kHalo + r;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (g < ng && t >= 0) x = *reinterpret_cast<const uint4*>(zx + t * a.ld_zx + a.col_x + (g0 + g) * VEC);
    xs[r][g] = x;
  }
  // dt of the x heads this slab touches
  const int c_lo = g0 * VEC, c_hi = min((g0 + ng) * VEC, a.d_inner);
  const int h_lo = c_lo / a.P, nh = c_hi > c_lo ? (c_hi - 1) / a.P - h_lo + 1 : 0;
  for (int j = tid; j < nt * nh; j += 256) {
    const int i = j / nh, hh = j % nh;
    dtS[i][hh] = softplus_f(E::to_f32(zx[(t0 + i) * a.ld_zx + a.col_dt + h_lo + hh]) + a.dt_bias[h_lo + hh]);
  }
  __syncthreads();

  const int g = tid % SG, tb = tid / SG;
  if (g >= ng) return;
  const int c0 = (g0 + g) * VEC;
  T* dst = nullptr;
  int h = 0;
  if (c0 < a.d_inner) {
    h = c0 / a.P;
    dst = static_cast<T*>(a.v) + ((bh0 + h) * a.T + t0) * a.P + c0 % a.P;
  } else {
    const bool isB = c0 < a.d_inner + a.G * a.N;
    const int cc = c0 - a.d_inner - (isB ? 0 : a.G * a.N);
    const int gi = cc / a.N;
    dst = static_cast<T*>(isB ? a.k : a.q) + (((size_t)b * a.G + gi) * a.T + t0) * a.N + cc % a.N;
  }
  const int row_len = c0 < a.d_inner ? a.P : a.N;
  float w[VEC][kMaxConvTaps], bias[VEC];
  load_taps<VEC>(a.taps, c0, w, bias);
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int i = 4 * tb + ii;
    if (i >= nt) break;
    float y[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) y[e] = bias[e];
#pragma unroll
    for (int j = 0; j < kMaxConvTaps; ++j) {
      float xv[VEC];
      const uint4 u = xs[i + j][g];
      if constexpr (BF16) {
        const unsigned w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xv[2 * e] = __builtin_bit_cast(float, w4[e] << 16);
          xv[2 * e + 1] = __builtin_bit_cast(float, w4[e] & 0xffff0000u);
        }
      } else {
        xv[0] = __builtin_bit_cast(float, u.x); xv[1] = __builtin_bit_cast(float, u.y);
        xv[2] = __builtin_bit_cast(float, u.z); xv[3] = __builtin_bit_cast(float, u.w);
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[e] = fmaf(w[e][j], xv[e], y[e]);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) y[e] = silu_f(y[e]);
    if (c0 < a.d_inner) {
      const float dt = dtS[i][h - h_lo];
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[e] *= dt;
    }
    store_vec<BF16, VEC>(dst + (size_t)i * row_len, y);
  }
}

// One workgroup per (sequence, kNormTokens tokens).  Thread (slot s,
// granule g) forms, for TR = kNormTokens / slots consecutive tokens, the
// x-channel conv + silu of granule g (taps from LDS), y = o + D x and the
// gated value y silu(z), and leaves its sum of squares in LDS; each wave then
// reduces (token, group) pairs, and the threads scale and store.
template <bool BF16, int TR>
__global__ __launch_bounds__(256) void mamba2_gate_norm(LayerArgs a) {
  using E = Elem<BF16>;
  using T = typename E::T;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int TOK = kNormTokens, SLOTS = TOK / TR, NR = TR + kHalo;
  __shared__ float part[TOK][256];
  __shared__ float rstd[TOK][256];
  const int b = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * TOK;
  const int nt = (int)min((int64_t)TOK, a.T - t0);
  const T* zx = static_cast<const T*>(a.zx) + (size_t)b * a.T * a.ld_zx;
  const int DG = a.d_inner / VEC;
  const int tid = threadIdx.x, g = tid % DG, s = tid / DG;
  const bool active = tid < SLOTS * DG;
  const int GG = DG / a.G;   // granules per norm group
  const int lane = tid & 63, w = tid >> 6;
  const int64_t ts = t0 + (int64_t)s * TR;
  const int n = active ? (int)max((int64_t)0, min((int64_t)TR, a.T - ts)) : 0;
  const int c0 = g * VEC, h = c0 / a.P;

  // this thread's inputs, all loads issued before any use: the conv window
  // (rows ts - kHalo .. ts + TR - 1, zero before the first token), z and o
  uint4 xr[NR], zr[TR], orr[TR];
  const T* oh = static_cast<const T*>(a.o) + (((size_t)b * a.H + h) * a.T) * a.P + c0 % a.P;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int64_t t = ts - kHalo + r;
    xr[r] = make_uint4(0, 0, 0, 0);
    if (n > 0 && t >= 0 && t < ts + n) xr[r] = *reinterpret_cast<const uint4*>(zx + t * a.ld_zx + a.col_x + c0);
  }
#pragma unroll
  for (int i = 0; i < TR; ++i) {
    zr[i] = make_uint4(0, 0, 0, 0);
    orr[i] = make_uint4(0, 0, 0, 0);
    if (i < n) {
      zr[i] = *reinterpret_cast<const uint4*>(zx + (ts + i) * a.ld_zx + c0);
      orr[i] = *reinterpret_cast<const uint4*>(oh + (ts + i) * a.P);
    }
  }
  float wt[VEC][kMaxConvTaps], bias[VEC];
  load_taps<VEC>(a.taps, c0, wt, bias);

  float gz[TR][VEC];
  if (n > 0) {
    const float Dh = a.D[h];
#pragma unroll
    for (int i = 0; i < TR; ++i) {
      float x[VEC], o[VEC], z[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[e] = bias[e];
#pragma unroll
      for (int j = 0; j < kMaxConvTaps; ++j) {
        float xv[VEC];
        unpack<BF16, VEC>(xr[i + j], xv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[e] = fmaf(wt[e][j], xv[e], x[e]);
      }
      unpack<BF16, VEC>(orr[i], o);
      unpack<BF16, VEC>(zr[i], z);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float v = (o[e] + Dh * silu_f(x[e])) * silu_f(z[e]);
        ss = fmaf(v, v, ss);
        gz[i][e] = v;
      }
      if (i < n) part[s * TR + i][g] = ss;
    }
  }
  __syncthreads();
  const float inv = 1.f / (float)(a.d_inner / a.G);
  for (int pr = w; pr < nt * a.G; pr += 4) {
    const int r = pr / a.G, gi = pr % a.G;
    float sum = 0.f;
    for (int j = lane; j < GG; j += 64) sum += part[r][gi * GG + j];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, 64);
    if (lane == 0) rstd[r][gi] = 1.f / sqrtf(sum * inv + a.eps);
  }
  __syncthreads();
  if (n > 0) {
    const int gi = g / GG;
    float nw[VEC];
    load_vec<BF16, VEC>(static_cast<const T*>(a.norm_w) + c0, nw);
    T* yrow = static_cast<T*>(a.y) + ((size_t)b * a.T) * a.d_inner + c0;
#pragma unroll
    for (int i = 0; i < TR; ++i) {
      if (i >= n) break;
      const float rs = rstd[s * TR + i][gi];
      float o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = gz[i][e] * rs * nw[e];
      store_vec<BF16, VEC>(yrow + (ts + i) * a.d_inner, o);
    }
  }
}

template <bool BF16>
int launch_gemm(const void* A, const void* B, void* C, int M, int N, int K, int lda, int ldb, int ldc,
                hipStream_t s) {
  if (M == 0 || N == 0) return kOK;
  const int64_t tiles_n = (N + kGemmTN - 1) / kGemmTN, tiles = (int64_t)((M + kGemmTM - 1) / kGemmTM) * tiles_n;
  if (tiles > 0x7fffffff) return kESHAPE;
  if ((int64_t)K * (BF16 ? 2 : 4) % (2 * kGemmKBytes) != 0) return kESHAPE;   // slices come in pairs
  if (ldc % (16 / (BF16 ? 2 : 4)) != 0) return kESHAPE;                          // 16-byte row pieces
  GemmArgs g{A, B, C, M, N, K, lda, ldb, ldc, (int)tiles_n, (int)tiles};
  const int lds = kGemmLds;
  if (hipFuncSetAttribute((const void*)gemm_nt<BF16>, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return kEHIP;
  hipLaunchKernelGGL((gemm_nt<BF16>), dim3((unsigned)tiles), dim3(256), lds, s, g);
  return hipGetLastError() == hipSuccess ? kOK : kEHIP;
}

// Input projection and the operator's inputs.
template <bool BF16>
int launch_layer_pre(const LayerPlan& p, const void* u, const void* in_proj, const LayerArgs& a, hipStream_t s) {
  int rc = launch_gemm<BF16>(u, in_proj, const_cast<void*>(a.zx), (int)p.M, p.d_in_proj, p.d_model, p.d_model,
                             p.d_model, p.ld_zx, s);
  if (rc != kOK) return rc;
  hipLaunchKernelGGL((mamba2_taps<BF16>), dim3((unsigned)((p.conv_dim + 255) / 256)), dim3(256), 0, s, a);
  const int n_slabs = (p.conv_dim / p.vec + kSlabGranules - 1) / kSlabGranules;
  const dim3 grid((unsigned)((p.T + kPrologueTokens - 1) / kPrologueTokens), (unsigned)p.B, (unsigned)(n_slabs + 1));
  hipLaunchKernelGGL((mamba2_prologue<BF16>), grid, dim3(256), 0, s, a, n_slabs);
  return hipGetLastError() == hipSuccess ? kOK : kEHIP;
}

// Gate, norm and output projection.
template <bool BF16>
int launch_layer_post(const LayerPlan& p, const void* out_proj, void* out, const LayerArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((p.T + kNormTokens - 1) / kNormTokens), (unsigned)p.B);
#define LA_GN(TR)                                                          \
  case TR:                                                                 \
    hipLaunchKernelGGL((mamba2_gate_norm<BF16, TR>), grid, dim3(256), 0, s, a); \
    break;
  switch (kNormTokens / p.norm_slots) {
    LA_GN(1) LA_GN(2) LA_GN(4) LA_GN(8) LA_GN(16)
    default: return kESHAPE;
  }
#undef LA_GN
  if (hipGetLastError() != hipSuccess) return kEHIP;
  return launch_gemm<BF16>(a.y, out_proj, out, (int)p.M, p.d_model, p.d_inner, p.d_inner, p.d_inner, p.d_model, s);
}

}  // namespace la
