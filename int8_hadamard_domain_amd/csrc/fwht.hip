// Blockwise 128-wide Walsh-Hadamard rotation of bf16 activation rows.
//
// The int8 card stores the experts' gate_up codes in the 128-wide Hadamard
// domain (model table, row "Weights"; recipe transform fwht128), so the
// activations take the same rotation before the product: y = H x / sqrt(128)
// per 128-block, H the Sylvester matrix in natural order.
//
// Mapping: 16 lanes per 128-block, 8 consecutive values per lane (one 16-byte
// load and store), 4 blocks per wavefront. Butterflies (a, b) -> (a+b, a-b)
// for index distance h: h = 1, 2, 4 run inside a lane; h = 8, 16, 32, 64 pair
// lane j with lane j^1, j^2, j^4, j^8 of the same 16-lane DPP row, moved with
// DPP (quad_perm for xor 1 and 2, row rotations for xor 4 and 8). All
// arithmetic is float32; one bf16 rounding at the end.

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

namespace i8h {

constexpr int kFwhtThreads = 256;
constexpr int kBlocksPerWg = kFwhtThreads / 16;

template <int M>
__device__ __forceinline__ void cross_stage(float (&v)[8], int j) {
  bool upper = (j & M) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float o = xor_lane<M>(v[i]);
    v[i] = upper ? (o - v[i]) : (v[i] + o);
  }
}

__global__ void __launch_bounds__(kFwhtThreads)
k_fwht128_bf16(const uint16_t* __restrict__ x, int64_t ldx, uint16_t* __restrict__ y, int64_t ldy,
               int T, int KB) {
  int64_t hb = (int64_t)blockIdx.x * kBlocksPerWg + threadIdx.x / 16;
  int j = threadIdx.x % 16;
  bool live = hb < (int64_t)T * KB;
  // every lane takes part in the cross-lane moves; dead lanes carry zeros
  int64_t t = live ? hb / KB : 0;
  int kb = live ? int(hb % KB) : 0;
  u32x4 w = {0u, 0u, 0u, 0u};
  if (live) w = *reinterpret_cast<const u32x4*>(x + t * ldx + kb * kGroup + 8 * j);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
  // in-lane stages h = 1, 2, 4
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  // cross-lane stages h = 8, 16, 32, 64
  cross_stage<1>(v, j);
  cross_stage<2>(v, j);
  cross_stage<4>(v, j);
  cross_stage<8>(v, j);
  const float rs = 0.08838834764831845f;  // 1/sqrt(128)
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(v[2 * i] * rs, v[2 * i + 1] * rs);
  if (live) *reinterpret_cast<u32x4*>(y + t * ldy + kb * kGroup + 8 * j) = o;
}

hipError_t launch_fwht128(const uint16_t* x, int64_t ldx, uint16_t* y, int64_t ldy, int T, int K,
                          hipStream_t st) {
  int KB = K / kGroup;
  int64_t nblk = (int64_t)T * KB;
  int grid = (int)((nblk + kBlocksPerWg - 1) / kBlocksPerWg);
  k_fwht128_bf16<<<grid, kFwhtThreads, 0, st>>>(x, ldx, y, ldy, T, KB);
  return hipGetLastError();
}

}  // namespace i8h
