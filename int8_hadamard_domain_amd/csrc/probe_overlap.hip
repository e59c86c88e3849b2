// Matrix-core / vector-ALU overlap probe: how much independent VALU work a
// wave can issue beside its MFMAs before the VALU, not the matrix pipe, sets
// the time. Not part of the product path (the probe library).
//
// Each wave runs four independent v_mfma_f32_32x32x16_bf16 accumulation
// chains and, after each MFMA, N independent float FMAs on registers of its
// own; scheduling barriers keep that order (MFMA, N FMAs, MFMA, ...) in the
// compiled loop. The caller times launches of one workgroup per CU with 256
// or 512 threads (one or two waves a SIMD); the time per MFMA and wave, as N
// grows, shows where the VALU stops hiding under the MFMAs. The results are
// summed into one word per thread so that nothing is removed.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/i8h_probe.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int N>
__device__ __forceinline__ void fmas(float (&v)[16], int first) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < N; ++j) v[(first + j) % 16] = fmaf(v[(first + j) % 16], 0.999f, 0.25f);
  __builtin_amdgcn_sched_barrier(0);
}

template <int N>
__global__ void __launch_bounds__(512) k_overlap_probe(float* __restrict__ out, int iters) {
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)(threadIdx.x % 7 + i);
    b[i] = (__bf16)(float)(i + 1);
  }
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = (float)(threadIdx.x + i);
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    fmas<N>(v, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    fmas<N>(v, 3);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    fmas<N>(v, 6);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    fmas<N>(v, 9);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i] + v[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" int i8h_overlap_probe(int nvalu, int threads, int blocks, int iters, float* out, void* stream) {
  if (!out || blocks <= 0 || iters <= 0 || (threads != 256 && threads != 512)) return -1;
  if ((reinterpret_cast<uintptr_t>(out) % 4) != 0) return -1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  switch (nvalu) {
    case 0: k_overlap_probe<0><<<blocks, threads, 0, st>>>(out, iters); break;
    case 2: k_overlap_probe<2><<<blocks, threads, 0, st>>>(out, iters); break;
    case 4: k_overlap_probe<4><<<blocks, threads, 0, st>>>(out, iters); break;
    case 6: k_overlap_probe<6><<<blocks, threads, 0, st>>>(out, iters); break;
    case 8: k_overlap_probe<8><<<blocks, threads, 0, st>>>(out, iters); break;
    case 12: k_overlap_probe<12><<<blocks, threads, 0, st>>>(out, iters); break;
    case 16: k_overlap_probe<16><<<blocks, threads, 0, st>>>(out, iters); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
