// Cross-lane moves within a 64-wide wavefront, picked per distance:
// DPP quad_perm for xor 1 and 2, ds_swizzle bit mode for xor 4 and 16,
// DPP row_ror:8 for xor 8 (a rotate by 8 inside a 16-lane row), and
// ds_bpermute for xor 32.
#pragma once

#include <hip/hip_runtime.h>

namespace i8h {

template <int M>
__device__ __forceinline__ int xor_lane_i(int i) {
  if constexpr (M == 1) i = __builtin_amdgcn_update_dpp(0, i, 0xB1, 0xF, 0xF, false);        // quad_perm 1,0,3,2
  else if constexpr (M == 2) i = __builtin_amdgcn_update_dpp(0, i, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  else if constexpr (M == 4) i = __builtin_amdgcn_ds_swizzle(i, (4 << 10) | 0x1F);           // bit mode, xor 4
  else if constexpr (M == 8) i = __builtin_amdgcn_update_dpp(0, i, 0x128, 0xF, 0xF, false);  // row_ror:8
  else if constexpr (M == 16) i = __builtin_amdgcn_ds_swizzle(i, (16 << 10) | 0x1F);         // bit mode, xor 16
  else i = __shfl_xor(i, 32, 64);
  return i;
}

template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  return __int_as_float(xor_lane_i<M>(__float_as_int(v)));
}

// Butterfly step of a Walsh-Hadamard transform across lanes at distance M:
// the lane with bit M clear keeps a + b, the other keeps a - b (a = lower).
template <int M>
__device__ __forceinline__ float hadamard_xlane(float v, int lane) {
  float o = xor_lane<M>(v);
  return (lane & M) ? (o - v) : (v + o);
}

}  // namespace i8h
