// Blockwise 128-wide Walsh-Hadamard rotation of bf16 activation rows.
//
// The int8 card stores the experts' gate_up codes in the 128-wide Hadamard
// domain (model table, row "Weights"; recipe transform fwht128), so the
// activations take the same rotation before the product: y = H x / sqrt(128)
// per 128-block, H the Sylvester matrix in natural order.
//
// Mapping: 16 lanes per 128-block, 8 consecutive values per lane (one 16-byte
// load and store), 4 blocks per wavefront; the block rotation itself is
// fwht128_block (rotate.hpp).

#include "common.hpp"
#include "launch.hpp"
#include "rotate.hpp"

namespace i8h {

constexpr int kFwhtThreads = 256;
constexpr int kBlocksPerWg = kFwhtThreads / 16;

__global__ void __launch_bounds__(kFwhtThreads)
k_fwht128_bf16(const uint16_t* x, int64_t ldx, uint16_t* y, int64_t ldy,   // in place allowed: not restrict
               int T, int KB) {
  int64_t hb = (int64_t)blockIdx.x * kBlocksPerWg + threadIdx.x / 16;
  int j = threadIdx.x % 16;
  bool live = hb < (int64_t)T * KB;
  // every lane takes part in the cross-lane moves; dead lanes carry zeros
  int64_t t = live ? hb / KB : 0;
  int kb = live ? int(hb % KB) : 0;
  u32x4 w = {0u, 0u, 0u, 0u};
  if (live) w = *reinterpret_cast<const u32x4*>(x + t * ldx + kb * kGroup + 8 * j);
  const u32x4 o = fwht128_block(w, j);
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
