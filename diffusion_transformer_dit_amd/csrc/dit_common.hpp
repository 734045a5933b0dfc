// Device-side helpers shared by the gfx950 kernels of libdit_block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// bf16 <-> fp32.  Widening is exact; narrowing is one v_cvt_pk_bf16_f32
// (round to nearest, ties to even) per pair of values.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint32_t f2bf_bits(float f) { return pack_bf2(f, 0.f) & 0xffffu; }

// 8 bf16 held in a 16-byte vector -> 8 floats
__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf_lo(v[i]);
    f[2 * i + 1] = bf_hi(v[i]);
  }
}
__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf2(f[2 * i], f[2 * i + 1]);
  return v;
}

// max / sum of the values held by lanes l and l^32, or l^16, on the lane-swap
// instructions (no LDS round trip): with both operands v, the swap's two
// results hold v and its partner, in an order that differs between the halves;
// max and sum do not depend on it (IEEE addition commutes).
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum / max over the 64 lanes of a wavefront (butterfly; every lane gets the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Fast transcendental building blocks on the hardware instructions.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// GELU, tanh form: 0.5 g (1 + tanh(u)) with u = sqrt(2/pi) (g + 0.044715 g^3).
// Since 0.5 (1 + tanh(u)) = 1 / (1 + e^{-2u}), this is g / (1 + 2^{-2u log2 e}),
// and -2u log2 e = g (k0 + k1 g^2) with the constants folded: 4 VALU + 2
// transcendentals + 1 add per value.
__device__ __forceinline__ float gelu_tanh(float g) {
  constexpr float k0 = -2.0f * kLog2e * 0.7978845608028654f;  // sqrt(2/pi)
  constexpr float k1 = k0 * 0.044715f;
  return g * rcp_fast(1.0f + exp2_fast(g * fmaf(k1, g * g, k0)));
}

__device__ __forceinline__ float silu(float z) { return z * rcp_fast(1.0f + exp2_fast(-kLog2e * z)); }

}  // namespace dit
