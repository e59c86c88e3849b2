// FP8 E4M3 128x128-block variant: the per-token, per-128 activation quantizer.
//
// Weights (FP8 card, model table row "Weights"): E4M3 codes per 128x128 block
// with one bf16 scale per block. The activations are bf16; FP8 MFMA needs
// FP8 operands, so they are quantized per token and per 128 of K with a
// float32 scale (the granularity of the int8 12B card's activations, header
// table row "Format"):
//   sx[t, g] = float32(amax / 448), qx = E4M3(x / sx) nearest even, saturating.
// Then
//   gu[r, n] = sum_g (sw[e, n/128, g] * sx[t, g]) * sum_{kk in g} qw * qx
//   act[r, i] = gelu_tanh(gu[r, i]) * gu[r, I + i].
//
// The E4M3 encoder is written out here (bit-exact, independent of the
// hardware convert's rounding and clamping modes): round the float32 to 3
// significand bits with ties to even, subnormals below 2^-6 in steps of 2^-9,
// magnitudes above 448 saturate, the sign bit is kept.
//
// Besides the codes and scales, the quantizer writes each code's exact value
// as bf16 (E4M3 has 3 significand bits): the grouped product consumes them
// on bf16 MFMA, where products are exact and sums are IEEE float32. (The
// gfx950 FP8 MFMA aligns its products to the largest one and keeps about 13
// bits below it, which misses a 1e-4 relative bound.)

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

namespace i8h {

// ---- activation quantizer ------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_from_f32(float v) {
  uint32_t bits = __float_as_uint(v);
  uint32_t sign = (bits >> 24) & 0x80u;
  uint32_t mag = bits & 0x7fffffffu;
  float a = __uint_as_float(mag);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: steps of 2^-9
    code = (uint32_t)rintf(a * 512.0f);      // exact scaling, nearest even; 8 -> 0x08
  } else if (a > 448.0f) {
    code = 0x7eu;
  } else {
    uint32_t q = mag >> 20;                  // fp32 exponent and top 3 significand bits
    uint32_t rem = mag & 0xfffffu;
    uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (q & 1u));
    code = q + up - (120u << 3);             // rebias exponent 127 -> 7
    if (code > 0x7eu) code = 0x7eu;
  }
  return sign | code;
}

// Exact bf16 bits of an E4M3 code: normal codes move their exponent and
// significand fields (rebias 7 -> 127); subnormal codes m * 2^-9 go through
// an exact float product.
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t c) {
  uint32_t sign = (c & 0x80u) << 8;
  uint32_t mag = c & 0x7fu;
  uint32_t bits;
  if (mag >= 8u) bits = (mag + (120u << 3)) << 4;
  else bits = __float_as_uint((float)mag * 0.001953125f) >> 16;  // m * 2^-9, exact
  return sign | bits;
}

constexpr int kQuantThreads = 256;

// 16 lanes per 128-value group, 8 values per lane.
__global__ void __launch_bounds__(kQuantThreads)
k_fp8_act_quant(const uint16_t* __restrict__ x, int T, int K, uint8_t* __restrict__ qx, float* __restrict__ sx,
                uint16_t* __restrict__ xq) {
  const int G = K / kGroup;
  int64_t grp = (int64_t)blockIdx.x * (kQuantThreads / 16) + threadIdx.x / 16;
  int j = threadIdx.x % 16;
  bool live = grp < (int64_t)T * G;
  int64_t t = live ? grp / G : 0;
  int g = live ? int(grp % G) : 0;
  u32x4 w = {0u, 0u, 0u, 0u};
  if (live) w = *reinterpret_cast<const u32x4*>(x + t * K + g * kGroup + 8 * j);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, xor_lane<1>(amax));
  amax = fmaxf(amax, xor_lane<2>(amax));
  amax = fmaxf(amax, xor_lane<4>(amax));
  amax = fmaxf(amax, xor_lane<8>(amax));
  float s = amax / 448.0f;                   // IEEE single division
  uint32_t out0 = 0, out1 = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out0 |= e4m3_from_f32(v[i] / s) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) out1 |= e4m3_from_f32(v[4 + i] / s) << (8 * i);
  }
  if (live) {
    *reinterpret_cast<u32x2*>(qx + t * K + g * kGroup + 8 * j) = u32x2{out0, out1};
    if (j == 0) sx[t * G + g] = s;
    if (xq) {
      u32x4 d;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        d[i] = e4m3_to_bf16((i < 2 ? out0 : out1) >> (16 * (i % 2)) & 0xffu) |
               (e4m3_to_bf16((i < 2 ? out0 : out1) >> (16 * (i % 2) + 8) & 0xffu) << 16);
      *reinterpret_cast<u32x4*>(xq + t * K + g * kGroup + 8 * j) = d;
    }
  }
}

hipError_t launch_fp8_act_quant(const uint16_t* x, int T, int K, uint8_t* qx, float* sx, uint16_t* xq,
                                hipStream_t st) {
  int64_t groups = (int64_t)T * (K / kGroup);
  int per = kQuantThreads / 16;
  int grid = (int)((groups + per - 1) / per);
  k_fp8_act_quant<<<grid, kQuantThreads, 0, st>>>(x, T, K, qx, sx, xq);
  return hipGetLastError();
}

}  // namespace i8h
