// Cross-lane moves within a 64-wide wavefront, all on the vector ALU (no LDS
// round trip, so a chain of them costs a few cycles per step instead of the
// LDS latency each):
//   xor 1, xor 2   DPP quad_perm
//   xor 4          DPP row_ror:4 (lanes with bit 2 set) or row_ror:12 (clear)
//   xor 8          DPP row_ror:8 (a rotation by 8 inside a 16-lane row)
//   xor 16         v_permlane16_swap (exchanges odd and even 16-lane rows)
//   xor 32         v_permlane32_swap (exchanges the two 32-lane halves)
// The swaps take the value twice (as "old" and "src") and return both
// exchanged copies; each lane keeps the one that came from its partner.
#pragma once

#include <hip/hip_runtime.h>

namespace i8h {

__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

template <int M>
__device__ __forceinline__ int xor_lane_i(int i) {
  if constexpr (M == 1) {
    return __builtin_amdgcn_update_dpp(0, i, 0xB1, 0xF, 0xF, false);    // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_update_dpp(0, i, 0x4E, 0xF, 0xF, false);    // quad_perm 2,3,0,1
  } else if constexpr (M == 4) {
    const int down = __builtin_amdgcn_update_dpp(0, i, 0x124, 0xF, 0xF, false);  // lane l <- l - 4 (row)
    const int up = __builtin_amdgcn_update_dpp(0, i, 0x12C, 0xF, 0xF, false);    // lane l <- l + 4 (row)
    return (lane_id() & 4) ? down : up;
  } else if constexpr (M == 8) {
    return __builtin_amdgcn_update_dpp(0, i, 0x128, 0xF, 0xF, false);   // row_ror:8
  } else if constexpr (M == 16) {
    const auto s = __builtin_amdgcn_permlane16_swap(i, i, false, false);
    return (lane_id() & 16) ? (int)s[0] : (int)s[1];
  } else {
    static_assert(M == 32, "xor distance must be 1, 2, 4, 8, 16 or 32");
    const auto s = __builtin_amdgcn_permlane32_swap(i, i, false, false);
    return (lane_id() & 32) ? (int)s[0] : (int)s[1];
  }
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

// Wave-wide float sum, butterfly over distances 32 .. 1 (fixed order, so
// every lane gets the same, deterministic value).
__device__ __forceinline__ float wave_sum(float v) {
  v += xor_lane<32>(v);
  v += xor_lane<16>(v);
  v += xor_lane<8>(v);
  v += xor_lane<4>(v);
  v += xor_lane<2>(v);
  v += xor_lane<1>(v);
  return v;
}

}  // namespace i8h
