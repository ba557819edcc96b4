// Device helpers for liblogattn (gfx950 only): element types, matrix-core
// wrappers, the Fenwick level function and wave-wide scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short bf16_t;   // storage type of a bfloat16 value

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(bf16_t u) {
  return __builtin_bit_cast(float, (unsigned)u << 16);
}
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// Element traits: storage type, matrix-core k-step and operand fragment.
//  bf16: v_mfma_f32_16x16x32_bf16 -- each lane supplies 8 consecutive k.
//  f32 : v_mfma_f32_16x16x4_f32   -- each lane supplies 1 k.
// In both, lane l supplies row/column (l % 16) of its operand and the k-slice
// indexed by (l / 16); the 16x16 fp32 result holds, in lane l, rows
// 4*(l/16) + i (i = 0..3) of column l % 16.
template <bool BF16> struct Elem;

template <> struct Elem<true> {
  using T = bf16_t;
  using Frag = bf16x8;
  static constexpr int kStep = 32;
  static constexpr int kPerLane = 8;
  static __device__ __forceinline__ float to_f32(T x) { return bf16_to_f32(x); }
  static __device__ __forceinline__ T from_f32(float x) { return f32_to_bf16(x); }
  // 8 consecutive elements starting at p (16-byte aligned).
  static __device__ __forceinline__ Frag load(const T* p) {
    return __builtin_bit_cast(Frag, *reinterpret_cast<const u16x8*>(p));
  }
  // Operand fragment whose k-slice starts at k0 in a contraction of length
  // K: zero when the slice lies past the end (K = 16 < kStep).
  template <int K>
  static __device__ __forceinline__ Frag load_k(const T* p, int k0) {
    if (K >= kStep || k0 < K) return load(p);
    return __builtin_bit_cast(Frag, u16x8{0, 0, 0, 0, 0, 0, 0, 0});
  }
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Elem<false> {
  using T = float;
  using Frag = float;
  static constexpr int kStep = 4;
  static constexpr int kPerLane = 1;
  static __device__ __forceinline__ float to_f32(T x) { return x; }
  static __device__ __forceinline__ T from_f32(float x) { return x; }
  static __device__ __forceinline__ Frag load(const T* p) { return *p; }
  template <int K>
  static __device__ __forceinline__ Frag load_k(const T* p, int) { return *p; }
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Fenwick bucket level of key j seen from query i inside one block of
// aligned positions (i >= j): 0 for the query itself, else 1 + the index of
// the highest bit where the two offsets differ.
__device__ __forceinline__ int fenwick_level_local(unsigned i, unsigned j) {
  return i == j ? 0 : 32 - __builtin_clz(i ^ j);
}

// Level of key s seen from query t with the chunk factorisation for chunk
// size 2^log2C; -1 when s > t.  Inside a chunk the level comes from the
// in-chunk offsets; across chunks it is log2C + 1 + msb(chunk_t ^ chunk_s).
__device__ __forceinline__ int fenwick_level(int64_t t, int64_t s, int log2C) {
  if (s > t) return -1;
  const int64_t ct = t >> log2C, cs = s >> log2C;
  if (ct == cs) {
    const unsigned mask = (1u << log2C) - 1u;
    return fenwick_level_local((unsigned)t & mask, (unsigned)s & mask);
  }
  return log2C + 1 + (63 - __builtin_clzll((unsigned long long)(ct ^ cs)));
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ float wave_incl_scan(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    float y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// The wave's index in its workgroup, as a wave-uniform (scalar) value: the
// compiler cannot tell that threadIdx.x / 64 is the same in every lane, and
// would otherwise keep it, and everything derived from it (tile indices,
// branches), in vector registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

}  // namespace la
