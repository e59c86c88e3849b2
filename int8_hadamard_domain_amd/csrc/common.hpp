// Shared device helpers for the gfx950 kernels of libi8h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8h {

constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kGroup = 128;    // K per scale group and per Hadamard block

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Signed byte j of a dword -> float (exact; v_cvt_f32_i32 with a sign-extended
// byte select).
template <int J>
__device__ __forceinline__ float sbyte(uint32_t w) {
  return (float)(int8_t)((w >> (8 * J)) & 0xffu);
}

// GELU, tanh approximation: v/2 (1 + tanh(z)) with z = sqrt(2/pi)(v + 0.044715 v^3).
// Evaluated as v / (1 + exp(-2z)), the same function written without the
// cancellation of 1 + tanh(z) for negative z, with the hardware base-2
// exponential and reciprocal (each about 1 ulp; exp(-2z) = 2^(-2 z log2 e),
// whose argument rounding adds a relative error of about |2z| 2^-24): a few
// float32 ulps in all, far inside the product's tolerance. Large |z| gives
// the exact limits (2^+big = inf -> v * 0, 2^-big = 0 -> v).
__device__ __forceinline__ float gelu_tanh(float v) {
  const float c2 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float t = c2 * (v + 0.044715f * v * v * v);
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

// One act value stored as float32, or as bf16 rounded to nearest even from that
// float32 value (the rounding the bf16 down projection applies to its input).
__device__ __forceinline__ void put_act(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void put_act(uint16_t* p, size_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, (__bf16)v);
}

__host__ __device__ constexpr inline int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace i8h
