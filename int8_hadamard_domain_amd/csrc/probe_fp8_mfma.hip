// FP8 matrix-core precision probe: runs gfx950's native E4M3 x E4M3 MFMA
// forms, and for contrast the bf16 form the FP8 grouped product uses, on
// caller data and writes the float32 results, so that a test can compare
// them with exact sums. It backs the choice of the FP8 grouped product
// (exact E4M3 -> bf16 decodes, bf16 MFMA) over the native FP8 instructions;
// it is not part of the product path (a separate library).
//
// One wave per 32x32 tile. A tile's operands are `steps` chunks; a chunk is
// the 64 lanes' operand registers, lane-major: `bpl` bytes per lane (32 for
// the 64-deep FP8 form, 8 for the 16-deep FP8 form, 16 = 8 bf16 values for
// the bf16 form). Lane l of a chunk holds the values of row l % 32 of A (of
// column l % 32 of B) for its half l / 32 of the contraction; both operands
// use the same half/element to k mapping, so a chunk contributes
//   C[m][n] += sum_{h<2} sum_{i} A[m + 32 h][i] * B[n + 32 h][i]
// whatever that mapping is. The chunks accumulate in order in the float32
// accumulator registers, as a K-loop of the product would.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/i8h_probe.h"

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

template <int FORM>
__global__ void __launch_bounds__(kWave)
k_fp8_mfma_probe(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b, float* __restrict__ c,
                 int steps) {
  constexpr int kBpl = FORM == 0 ? 32 : FORM == 1 ? 8 : 16;
  const int lane = threadIdx.x;
  const size_t tile = blockIdx.x;
  const size_t chunk = (size_t)kWave * kBpl;
  const uint8_t* at = a + tile * steps * chunk + (size_t)lane * kBpl;
  const uint8_t* bt = b + tile * steps * chunk + (size_t)lane * kBpl;
  f32x16 acc = {};
  for (int s = 0; s < steps; ++s) {
    if constexpr (FORM == 0) {
      const i32x8 av = *reinterpret_cast<const i32x8*>(at + s * chunk);
      const i32x8 bv = *reinterpret_cast<const i32x8*>(bt + s * chunk);
      // format codes 0/0: both operands E4M3; zero scale operands select the
      // unscaled instruction
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
    } else if constexpr (FORM == 1) {
      const long av = *reinterpret_cast<const long*>(at + s * chunk);
      const long bv = *reinterpret_cast<const long*>(bt + s * chunk);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(av, bv, acc, 0, 0, 0);
    } else {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(at + s * chunk);
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(bt + s * chunk);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    }
  }
  // 32x32 accumulator layout: register r of lane l holds
  // C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]
  float* ct = c + tile * 1024;
#pragma unroll
  for (int r = 0; r < 16; ++r) ct[(8 * (r / 4) + 4 * (lane / 32) + r % 4) * 32 + lane % 32] = acc[r];
}

}  // namespace

extern "C" int i8h_fp8_mfma_probe(int form, const void* a, const void* b, float* c, int tiles, int steps,
                                  void* stream) {
  if (form < 0 || form > 2 || !a || !b || !c || tiles <= 0 || steps <= 0) return -1;
  const uintptr_t align = form == 0 ? 32 : form == 1 ? 8 : 16;
  if ((reinterpret_cast<uintptr_t>(a) % align) != 0 || (reinterpret_cast<uintptr_t>(b) % align) != 0 ||
      (reinterpret_cast<uintptr_t>(c) % 4) != 0)
    return -1;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* pa = static_cast<const uint8_t*>(a);
  const uint8_t* pb = static_cast<const uint8_t*>(b);
  if (form == 0)
    k_fp8_mfma_probe<0><<<tiles, kWave, 0, st>>>(pa, pb, c, steps);
  else if (form == 1)
    k_fp8_mfma_probe<1><<<tiles, kWave, 0, st>>>(pa, pb, c, steps);
  else
    k_fp8_mfma_probe<2><<<tiles, kWave, 0, st>>>(pa, pb, c, steps);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
