// Shared device helpers for the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // storage type of a bf16 value

constexpr int kWave = 64;
constexpr int kExperts = 8;
constexpr int kTopK = 2;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float v) {
  __bf16 b = static_cast<__bf16>(v);
  return __builtin_bit_cast(bf16_t, b);
}

// Two floats -> two packed bf16 (low half = a), one v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// SiLU(z) = z * sigmoid(z) with the hardware exp2 and reciprocal (about 1 ulp
// each, far below the bf16 rounding of h); z -> -inf gives -0, +inf gives z.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// One output element of the gate-weighted combine, the two slots added in
// slot order: g0*a + g1*b, a dropped slot (k = false) adding nothing.  Each
// operation rounds once (no contraction into a fused multiply-add), so every
// kernel that combines gives the same bits.
__device__ __forceinline__ float combine_pair(float a, float b, float g0, float g1, bool k0, bool k1) {
  return __fadd_rn(k0 ? __fmul_rn(g0, a) : 0.0f, k1 ? __fmul_rn(g1, b) : 0.0f);
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Find the expert owning global m-tile `mt` given per-expert row counts in
// offsets[0..E]; returns -1 when mt is past the last tile.  `bm` = tile rows.
__device__ __forceinline__ int locate_m_tile(const int32_t* offs, int mt, int bm, int* m0_out,
                                             int* row_begin, int* rows) {
  int acc = 0;
#pragma unroll
  for (int e = 0; e < kExperts; ++e) {
    const int beg = offs[e];
    const int cnt = offs[e + 1] - beg;
    const int tiles = (cnt + bm - 1) / bm;
    if (mt < acc + tiles) {
      *m0_out = (mt - acc) * bm;
      *row_begin = beg;
      *rows = cnt;
      return e;
    }
    acc += tiles;
  }
  return -1;
}

}  // namespace moe
