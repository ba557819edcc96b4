// Recurrent decode step, decode-state initialisation and the level-table
// export for liblogattn (gfx950).
//
// Decode ("Log-Linear Attention", Italian summary, technical section 2,
// item 3 "Decoding"; lay part "L'essenziale": only the smallest box is
// updated and, when needed, merged into the bigger ones): one d_k x d_v fp32
// state per Fenwick level; at position t the levels whose bit is set in t are
// occupied.  The gate is applied lazily to a per-slot scalar so that a step
// streams only the occupied slots once and writes one merged slot.
#include "la_device.hpp"
#include "la_internal.hpp"
#include "la_levels.hpp"
#include "la_plan.hpp"

namespace la {

struct DecArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* lam;
  void* out;
  float* slots;   // [BH][S][D][D]
  float* scale;   // [BH][S]
  int64_t t;
  int S;
  int kstar;      // trailing ones of t: levels 1..kstar merge into kstar+1
};

template <bool BF16, int D>
__global__ __launch_bounds__(256) void decode_step_kernel(DecArgs x) {
  using EL = Elem<BF16>;
  using E = typename EL::T;
  constexpr int NT = (D * D / 4) < 256 ? (D * D / 4) : 256;   // threads streaming the slots
  constexpr int C4 = D / 4;                                   // float4 per row
  constexpr int RG = NT / C4;                                 // row groups
  constexpr int RPT = D / RG;                                 // rows per thread
  __shared__ float qs[D], ks[D], vs[D], lam_s[kMaxDecodeSlots + 1], sc_s[kMaxDecodeSlots];
  __shared__ float red[RG][D];
  __shared__ float qk_s;

  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int S = x.S;
  const int64_t t = x.t;
  const float at = x.a[bh];
  const E* qg = reinterpret_cast<const E*>(x.q) + bh * D;
  const E* kg = reinterpret_cast<const E*>(x.k) + bh * D;
  const E* vg = reinterpret_cast<const E*>(x.v) + bh * D;
  if (tid < D) {
    qs[tid] = EL::to_f32(qg[tid]);
    ks[tid] = EL::to_f32(kg[tid]);
    vs[tid] = EL::to_f32(vg[tid]);
  }
  if (tid <= S) lam_s[tid] = x.lam[bh * (S + 1) + tid];
  if (tid < S) sc_s[tid] = x.scale[bh * S + tid];
  __syncthreads();

  if (tid < 64) {   // q . k, fixed-order butterfly (deterministic)
    float p = 0.f;
    for (int j = tid; j < D; j += 64) p += qs[j] * ks[j];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) p += __shfl_xor(p, o, 64);
    if (tid == 0) qk_s = p;
  }

  const int c4 = tid % C4, rg = tid / C4;
  float4 op = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 m[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) m[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* sb = x.slots + bh * (int64_t)S * D * D;
  if (tid < NT) {
    for (int l = 1; l <= S; ++l) {
      if (!((t >> (l - 1)) & 1)) continue;        // level l empty at position t
      const float sc = sc_s[l - 1] * at;          // gate of this token applied
      const float wgt = lam_s[l] * sc;
      const bool merge = l <= x.kstar;
      const float* sl = sb + (int64_t)(l - 1) * D * D;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        const float4 s4 = *reinterpret_cast<const float4*>(sl + row * D + 4 * c4);
        const float wq = wgt * qs[row];
        op.x += wq * s4.x; op.y += wq * s4.y; op.z += wq * s4.z; op.w += wq * s4.w;
        if (merge) {
          m[i].x += sc * s4.x; m[i].y += sc * s4.y; m[i].z += sc * s4.z; m[i].w += sc * s4.w;
        }
      }
    }
    // merged bucket: this token plus levels 1..kstar, at level kstar+1
    float* dst = x.slots + (bh * (int64_t)S + x.kstar) * D * D;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg + RG * i;
      const float kr = ks[row];
      float4 nv;
      nv.x = m[i].x + kr * vs[4 * c4 + 0];
      nv.y = m[i].y + kr * vs[4 * c4 + 1];
      nv.z = m[i].z + kr * vs[4 * c4 + 2];
      nv.w = m[i].w + kr * vs[4 * c4 + 3];
      *reinterpret_cast<float4*>(dst + row * D + 4 * c4) = nv;
    }
    red[rg][4 * c4 + 0] = op.x;
    red[rg][4 * c4 + 1] = op.y;
    red[rg][4 * c4 + 2] = op.z;
    red[rg][4 * c4 + 3] = op.w;
  }
  __syncthreads();
  if (tid < D) {
    float o = lam_s[0] * qk_s * vs[tid];
    for (int r = 0; r < RG; ++r) o += red[r][tid];
    reinterpret_cast<E*>(x.out)[bh * D + tid] = EL::from_f32(o);
  }
  if (tid < S) {
    const int l = tid + 1;
    if (l == x.kstar + 1) x.scale[bh * S + tid] = 1.f;
    else if ((t >> (l - 1)) & 1) x.scale[bh * S + tid] = sc_s[tid] * at;
  }
}

__global__ void state_init_kernel(float* slots, int64_t n_slots, float* scale, int64_t n_scale) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_slots; i += stride) slots[i] = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_scale; i += stride) scale[i] = 1.f;
}

__global__ void level_table_kernel(int64_t T, int log2C, int8_t* out) {
  const int64_t n = T * T;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t t = i / T, s = i % T;
    // inside a chunk from the chunk-relative offsets, across chunks through
    // the output kernel's bucket enumeration (groups of eight chunks)
    const int64_t ct = t >> log2C, cs = s >> log2C;
    out[i] = (int8_t)(s > t ? -1 : ct == cs ? fenwick_level(t, s, log2C)
                                            : enumerated_chunk_level(ct, cs, log2C, ilog2(state_group(64))));
  }
}

template <bool BF16>
static int launch_decode_d(int D, DecArgs a, int64_t BH, hipStream_t s) {
  switch (D) {
    case 16: hipLaunchKernelGGL((decode_step_kernel<BF16, 16>), dim3((unsigned)BH), dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((decode_step_kernel<BF16, 32>), dim3((unsigned)BH), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((decode_step_kernel<BF16, 64>), dim3((unsigned)BH), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL((decode_step_kernel<BF16, 128>), dim3((unsigned)BH), dim3(256), 0, s, a); break;
    default: return kESHAPE;
  }
  return hipGetLastError() == hipSuccess ? kOK : kEHIP;
}

int launch_decode(const la_state* st, const void* q, const void* k, const void* v, const float* a,
                  const float* lam, void* out, int dtype, int kstar, hipStream_t s) {
  DecArgs x{q, k, v, a, lam, out, st->slots, st->scale, st->t, st->S, kstar};
  const int64_t BH = (int64_t)st->B * st->H;
  return dtype == kBF16 ? launch_decode_d<true>(st->dk, x, BH, s) : launch_decode_d<false>(st->dk, x, BH, s);
}

int launch_state_init(float* slots, int64_t n_slots, float* scale, int64_t n_scale, hipStream_t s) {
  int64_t blocks = (n_slots + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(state_init_kernel, dim3((unsigned)blocks), dim3(256), 0, s, slots, n_slots, scale, n_scale);
  return hipGetLastError() == hipSuccess ? kOK : kEHIP;
}

int launch_level_table(int64_t T, int log2C, int8_t* out, hipStream_t s) {
  int64_t blocks = (T * T + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(level_table_kernel, dim3((unsigned)blocks), dim3(256), 0, s, T, log2C, out);
  return hipGetLastError() == hipSuccess ? kOK : kEHIP;
}

}  // namespace la
