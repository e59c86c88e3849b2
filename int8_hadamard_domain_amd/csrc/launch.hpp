// Internal launchers, called by the C ABI after host-side validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace i8h {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopk = 32;

// chunks of whole tokens (at most 256 pairs each) of the many-token routing
int64_t route_chunks(int T, int k);
size_t route_workspace_bytes(int T, int E, int k);
// the allocation-free routing call's device scratch: its size, and its
// address on the current device (which must be the stream's), looked up once
// per device
constexpr size_t kRouteScratchBytes = (size_t)1 << 20;
hipError_t route_scratch(hipStream_t st, void** out);
// x != NULL also rotates the T activation rows x [T, K] into xr (x may be xr)
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        int32_t* expert_off, int32_t* sorted_pairs, int32_t* pair_pos,
                        void* ws, const uint16_t* x, uint16_t* xr, int K, hipStream_t st);

hipError_t launch_fwht128(const uint16_t* x, int64_t ldx, uint16_t* y, int64_t ldy, int T, int K,
                          hipStream_t st);

// gate_up launchers: act is float32 [P, I], or bf16 [P, I] when act_bf16 (each
// value rounded to nearest even from the float32 one)
hipError_t launch_gateup_i8h_gemv(const uint16_t* xrot, int T, int K, const int8_t* codes,
                                  const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                  const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16,
                                  hipStream_t st);
hipError_t launch_gateup_i8h_gemm(const uint16_t* xrot, int T, int K, const int8_t* codes,
                                  const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                  const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16,
                                  hipStream_t st);

hipError_t launch_gateup_i8h_gemm_tall(const uint16_t* xrot, int T, int K, const int8_t* codes,
                                       const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                       const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16,
                                       hipStream_t st);

hipError_t launch_gateup_i8h_skinny(const uint16_t* xrot, int T, int K, const int8_t* codes,
                                    const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                    const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16,
                                    hipStream_t st);

hipError_t launch_gateup_fp8_skinny(const uint16_t* xq, const float* sx, int T, int K, const uint8_t* codes,
                                    const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                    const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16,
                                    hipStream_t st);

hipError_t launch_i8_act_quant(const uint16_t* x, int T, int K, int8_t* qx, float* sx, hipStream_t st);

hipError_t launch_gateup_i8g(const int8_t* qx, const float* sx, int T, int K, const int8_t* codes,
                             const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                             const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16,
                             hipStream_t st);

hipError_t launch_gateup_i8h_gemv_rot(const uint16_t* x, int T, int K, const int8_t* codes,
                                      const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                      const int32_t* sorted_pairs, float* gu, float* act, hipStream_t st);

hipError_t launch_route_gateup_decode(const float* logits, const uint16_t* x, int T, int K, const int8_t* codes,
                                      const uint16_t* scales, int E, int N, int k, int32_t* ids, float* w,
                                      int32_t* expert_off, int32_t* sorted_pairs, int32_t* pair_pos, float* gu,
                                      float* act, hipStream_t st);

hipError_t launch_fp8_act_quant(const uint16_t* x, int T, int K, uint8_t* qx, float* sx, uint16_t* xq,
                                hipStream_t st);
hipError_t launch_gateup_fp8(const uint16_t* xq, const float* sx, int T, int K, const uint8_t* codes,
                             const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                             const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16,
                             hipStream_t st);

// bf16 grouped down projection + weighted combine (down.hip); act is float32
// [P, I], or bf16 [P, I] when act_bf16 (then a16 is not used)
hipError_t launch_down_gemv_combine(const void* act, bool act_bf16, int T, int I, const uint16_t* w, int H, int k,
                                    const int32_t* ids, const float* tw, const int32_t* pos, float* out,
                                    hipStream_t st);
hipError_t launch_down_gemm_combine(const void* act, bool act_bf16, int T, int I, const uint16_t* w, int E, int H,
                                    int k, const float* tw, const int32_t* expert_off, const int32_t* pos,
                                    uint16_t* a16, float* y, float* out, hipStream_t st);

// dense int8 linear with f16 group scales (linear.hip)
hipError_t launch_linear_i8f16(const uint16_t* x, int T, int K, const int8_t* codes, const uint16_t* scales, int N,
                               float* y, hipStream_t st);

}  // namespace i8h
