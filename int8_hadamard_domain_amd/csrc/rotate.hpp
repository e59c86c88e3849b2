// The 128-wide Walsh-Hadamard rotation of one 128-value block held by 16
// lanes (8 consecutive values each), shared by the rotation kernel and the
// routing kernel that rotates the token rows it routes: y = H x / sqrt(128),
// H the Sylvester matrix in natural order (the int8 card's 128-wide Hadamard
// domain, model table row "Weights"; recipe transform fwht128).
//
// Butterflies (a, b) -> (a+b, a-b) for index distance h: h = 1, 2, 4 inside a
// lane; h = 8, 16, 32, 64 pair lane j with lane j^1, j^2, j^4, j^8 of the same
// 16-lane DPP row (quad_perm for xor 1 and 2, row rotations for xor 4 and 8).
// All arithmetic is float32, in this fixed order; one bf16 rounding at the
// end, so every caller produces the same bits.
#pragma once

#include "common.hpp"
#include "xlane.hpp"

namespace i8h {

template <int M>
__device__ __forceinline__ void fwht_cross_stage(float (&v)[8], int j) {
  const bool upper = (j & M) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = xor_lane<M>(v[i]);
    v[i] = upper ? (o - v[i]) : (v[i] + o);
  }
}

// w: the lane's 8 bf16 values (positions 8 j .. 8 j + 7 of the block, j =
// lane % 16); returns the rotated values rounded to bf16, packed the same way.
// Every lane of the 16-lane row must call it (dead lanes pass zeros).
__device__ __forceinline__ u32x4 fwht128_block(const u32x4 w, int j) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  fwht_cross_stage<1>(v, j);
  fwht_cross_stage<2>(v, j);
  fwht_cross_stage<4>(v, j);
  fwht_cross_stage<8>(v, j);
  const float rs = 0.08838834764831845f;  // 1/sqrt(128)
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(v[2 * i] * rs, v[2 * i + 1] * rs);
  return o;
}

}  // namespace i8h
