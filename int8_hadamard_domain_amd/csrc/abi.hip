// C ABI of libi8h: host-side validation, kernel choice and launch.
// Every check runs before any HIP call, so an invalid call has no effect.

#include <hip/hip_runtime.h>

#include "../../include/i8h.h"
#include "launch.hpp"

namespace {

using i8h::kMaxExperts;
using i8h::kMaxTopk;

constexpr int kGemvMaxK = 4096;   // the decode kernel keeps K/1024 pieces per lane
constexpr int kGemvMaxT = 8;      // AUTO picks the decode kernel up to this many tokens
constexpr int kDecodeMaxPairs = 64;     // the fused decode kernel groups all pairs in one wave
constexpr int kDecodeMaxExperts = 256;  // ... and ranks at most 4 logits per lane

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int from_hip(hipError_t e) { return e == hipSuccess ? I8H_OK : I8H_EHIP; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_common_moe(int T, int K, int E, int N, int topk) {
  if (T < 0 || K <= 0 || (K % 128) != 0 || E <= 0 || N <= 0 || topk <= 0) return I8H_EINVAL;
  if (E > kMaxExperts || topk > kMaxTopk || topk > E) return I8H_EUNSUPPORTED;
  if ((int64_t)T * topk >= (int64_t)1 << 31) return I8H_EUNSUPPORTED;
  if ((int64_t)T * K >= (int64_t)1 << 31) return I8H_EUNSUPPORTED;  // activation offsets are 32-bit
  return I8H_OK;
}

inline bool auto_gemv(int T, int K) { return T <= kGemvMaxT && K <= kGemvMaxK; }

// the tall kernel addresses one expert's codes with 32-bit offsets
inline bool tall_fits(int K, int N) { return (int64_t)N * K < ((int64_t)1 << 31); }

// kernel for the MFMA range: 256-pair passes once experts average 32 pairs,
// below that the small-unit kernel (64-pair passes, three workgroups a CU)
inline int auto_path(int T, int K, int E, int N, int topk) {
  if (auto_gemv(T, K)) return I8H_PATH_GEMV;
  if ((int64_t)T * topk >= (int64_t)32 * E && tall_fits(K, N)) return I8H_PATH_TALL;
  return I8H_PATH_SKINNY;
}

// act: float32 [P, I], or bf16 [P, I] when act_bf16
int gateup_i8h(const uint16_t* x_rot, int T, int K, const int8_t* codes, const uint16_t* scales, int E, int N,
               int topk, const int32_t* expert_off, const int32_t* sorted_pairs, float* gate_up, void* act,
               bool act_bf16, int path, void* stream) {
  int rc = check_common_moe(T, K, E, N, topk);
  if (rc != I8H_OK) return rc;
  if ((N % 2) != 0) return I8H_EINVAL;                  // gate and up halves
  if ((N % 64) != 0) return I8H_EUNSUPPORTED;           // 32-row gate and up tiles
  if (path < I8H_PATH_AUTO || path > I8H_PATH_SKINNY) return I8H_EINVAL;
  if (T == 0) return I8H_OK;
  if (!x_rot || !codes || !scales || !expert_off || !sorted_pairs) return I8H_EINVAL;
  if (!aligned(x_rot, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return I8H_EINVAL;
  if (!aligned(expert_off, 4) || !aligned(sorted_pairs, 4)) return I8H_EINVAL;
  if ((gate_up && !aligned(gate_up, 4)) || (act && !aligned(act, act_bf16 ? 2 : 4))) return I8H_EINVAL;
  if (!gate_up && !act) return I8H_OK;  // nothing requested
  if (path == I8H_PATH_GEMV && K > kGemvMaxK) return I8H_EUNSUPPORTED;
  if (path == I8H_PATH_TALL && !tall_fits(K, N)) return I8H_EUNSUPPORTED;
  if (path == I8H_PATH_AUTO) path = auto_path(T, K, E, N, topk);
  hipError_t e;
  if (path == I8H_PATH_GEMV)
    e = i8h::launch_gateup_i8h_gemv(x_rot, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs, gate_up,
                                    act, act_bf16, as_stream(stream));
  else if (path == I8H_PATH_TALL)
    e = i8h::launch_gateup_i8h_gemm_tall(x_rot, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs,
                                         gate_up, act, act_bf16, as_stream(stream));
  else if (path == I8H_PATH_SKINNY)
    e = i8h::launch_gateup_i8h_skinny(x_rot, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs, gate_up,
                                      act, act_bf16, as_stream(stream));
  else
    e = i8h::launch_gateup_i8h_gemm(x_rot, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs, gate_up,
                                    act, act_bf16, as_stream(stream));
  return from_hip(e);
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// FP8 workspace: qx [T, K] uint8, sx [T, K/128] float32, xq [T, K] bf16
struct Fp8Ws {
  size_t sx_off, xq_off, total;
  Fp8Ws(int T, int K) {
    sx_off = round_up((size_t)T * K, 256);
    xq_off = sx_off + round_up((size_t)T * (K / 128) * sizeof(float), 256);
    total = xq_off + round_up((size_t)T * K * 2, 256);
  }
};

// W8A8 workspace: qx [T, K] int8, sx [T, K/128] float32
size_t i8g_sx_off(int T, int K) { return round_up((size_t)T * K, 256); }
size_t i8g_ws_total(int T, int K) {
  return i8g_sx_off(T, K) + round_up((size_t)T * (K / 128) * sizeof(float), 256);
}

}  // namespace

// bf16 grouped down projection + weighted combine
namespace {

constexpr int kDownGemvMaxPairs = 64;   // AUTO: the one-launch form up to this many pairs
constexpr int kDownGemvMaxI = 1024;     // the one-launch form keeps I/256 pieces per lane

inline bool down_gemv_ok(int I, int H) { return I <= kDownGemvMaxI && (H % 8) == 0; }
inline bool down_gemm_ok(int T, int I, int H, int topk) {
  return (I % 32) == 0 && I >= 96 && (H % 256) == 0 && (int64_t)T * topk * I < ((int64_t)1 << 31) &&
         (int64_t)256 * I < ((int64_t)1 << 31);
}

struct DownWs {
  size_t a16, y, total;
  DownWs(int T, int I, int H, int topk) {
    const size_t p = (size_t)T * topk;
    a16 = round_up(p * I * 2, 256);
    y = round_up(p * H * 4, 256);
    total = a16 + y;
  }
};

// act: float32 [P, I], or bf16 [P, I] when act_bf16 (then the workspace holds y only)
int down_combine(const void* act, bool act_bf16, int T, int I, const uint16_t* w_down, int E, int H, int topk,
                 const int32_t* topk_ids, const float* topk_w, const int32_t* expert_off, const int32_t* pair_pos,
                 float* out, void* workspace, size_t workspace_bytes, int path, void* stream) {
  if (T < 0 || I <= 0 || (I % 8) != 0 || H <= 0 || (H % 8) != 0 || E <= 0 || topk <= 0) return I8H_EINVAL;
  if (E > kMaxExperts || topk > kMaxTopk || topk > E) return I8H_EUNSUPPORTED;
  if ((int64_t)T * topk >= (int64_t)1 << 31) return I8H_EUNSUPPORTED;
  if (path < I8H_DOWN_AUTO || path > I8H_DOWN_GEMM) return I8H_EINVAL;
  if (T == 0) return I8H_OK;
  if (!act || !w_down || !topk_ids || !topk_w || !expert_off || !pair_pos || !out) return I8H_EINVAL;
  if (!aligned(act, 16) || !aligned(w_down, 16) || !aligned(out, 16)) return I8H_EINVAL;
  if (!aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(expert_off, 4) || !aligned(pair_pos, 4))
    return I8H_EINVAL;
  const int64_t pairs = (int64_t)T * topk;
  if (path == I8H_DOWN_AUTO) {
    if (pairs <= kDownGemvMaxPairs && down_gemv_ok(I, H)) path = I8H_DOWN_GEMV;
    else if (down_gemm_ok(T, I, H, topk)) path = I8H_DOWN_GEMM;
    else if (down_gemv_ok(I, H)) path = I8H_DOWN_GEMV;
    else return I8H_EUNSUPPORTED;
  }
  if (path == I8H_DOWN_GEMV) {
    if (!down_gemv_ok(I, H)) return I8H_EUNSUPPORTED;
    return from_hip(i8h::launch_down_gemv_combine(act, act_bf16, T, I, w_down, H, topk, topk_ids, topk_w, pair_pos,
                                                  out, as_stream(stream)));
  }
  if (!down_gemm_ok(T, I, H, topk)) return I8H_EUNSUPPORTED;
  const DownWs ws(T, I, H, topk);
  const size_t need = act_bf16 ? ws.y : ws.total;
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return I8H_EINVAL;
  uint8_t* base = static_cast<uint8_t*>(workspace);
  uint16_t* a16 = act_bf16 ? nullptr : reinterpret_cast<uint16_t*>(base);
  float* y = reinterpret_cast<float*>(act_bf16 ? base : base + ws.a16);
  return from_hip(i8h::launch_down_gemm_combine(act, act_bf16, T, I, w_down, E, H, topk, topk_w, expert_off,
                                                pair_pos, a16, y, out, as_stream(stream)));
}

}  // namespace

extern "C" {

const char* i8h_status_string(int status) {
  switch (status) {
    case I8H_OK: return "ok";
    case I8H_EINVAL: return "invalid argument";
    case I8H_EUNSUPPORTED: return "unsupported size";
    case I8H_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

size_t moe_route_permute_workspace_size(int T, int E, int topk) {
  if (T <= 0 || E <= 0 || topk <= 0 || E > kMaxExperts || topk > kMaxTopk) return 0;
  return i8h::route_workspace_bytes(T, E, topk);
}

int moe_route_permute(const float* logits, int T, int E, int topk, int32_t* topk_ids, float* topk_w,
                      int32_t* expert_off, int32_t* sorted_pairs, int32_t* pair_pos, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (T < 0 || E <= 0 || topk <= 0) return I8H_EINVAL;
  if (E > kMaxExperts || topk > kMaxTopk || topk > E) return I8H_EUNSUPPORTED;
  if ((int64_t)T * topk >= (int64_t)1 << 31) return I8H_EUNSUPPORTED;
  // the chunk histograms (E counts per chunk of whole tokens) are indexed in 32 bits
  if (i8h::route_chunks(T, topk) * E >= (int64_t)1 << 31) return I8H_EUNSUPPORTED;
  if (T == 0) return I8H_OK;
  if (!logits || !topk_ids || !topk_w || !expert_off || !sorted_pairs || !pair_pos) return I8H_EINVAL;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(expert_off, 4) ||
      !aligned(sorted_pairs, 4) || !aligned(pair_pos, 4))
    return I8H_EINVAL;
  size_t need = i8h::route_workspace_bytes(T, E, topk);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 4))) return I8H_EINVAL;
  return from_hip(i8h::launch_route(logits, T, E, topk, topk_ids, topk_w, expert_off, sorted_pairs, pair_pos,
                                    workspace, nullptr, nullptr, 0, as_stream(stream)));
}

int moe_route_permute_rotate(const float* logits, const uint16_t* x, int T, int E, int topk, int K,
                             int32_t* topk_ids, float* topk_w, int32_t* expert_off, int32_t* sorted_pairs,
                             int32_t* pair_pos, uint16_t* x_rot, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (T < 0 || E <= 0 || topk <= 0 || K <= 0 || (K % 128) != 0) return I8H_EINVAL;
  if (E > kMaxExperts || topk > kMaxTopk || topk > E) return I8H_EUNSUPPORTED;
  if ((int64_t)T * topk >= (int64_t)1 << 31) return I8H_EUNSUPPORTED;
  if ((int64_t)T * K >= (int64_t)1 << 31) return I8H_EUNSUPPORTED;     // activation offsets
  if (i8h::route_chunks(T, topk) * E >= (int64_t)1 << 31) return I8H_EUNSUPPORTED;
  if (T == 0) return I8H_OK;
  if (!logits || !x || !x_rot || !topk_ids || !topk_w || !expert_off || !sorted_pairs || !pair_pos)
    return I8H_EINVAL;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(expert_off, 4) ||
      !aligned(sorted_pairs, 4) || !aligned(pair_pos, 4) || !aligned(x, 16) || !aligned(x_rot, 16))
    return I8H_EINVAL;
  if (x != x_rot) {
    // other overlap would let one row's rotation read what another already wrote
    uintptr_t xb = reinterpret_cast<uintptr_t>(x), yb = reinterpret_cast<uintptr_t>(x_rot);
    uintptr_t bytes = 2 * (uintptr_t)((int64_t)T * K);
    if (xb < yb + bytes && yb < xb + bytes) return I8H_EINVAL;
  }
  size_t need = i8h::route_workspace_bytes(T, E, topk);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 4))) return I8H_EINVAL;
  return from_hip(i8h::launch_route(logits, T, E, topk, topk_ids, topk_w, expert_off, sorted_pairs, pair_pos,
                                    workspace, x, x_rot, K, as_stream(stream)));
}

int moe_route_permute_noalloc(const float* logits, int T, int E, int topk, int32_t* topk_ids, float* topk_w,
                              int32_t* expert_off, int32_t* sorted_pairs, int32_t* pair_pos, void* stream) {
  // the checks of moe_route_permute, then the scratch size instead of a workspace
  if (T < 0 || E <= 0 || topk <= 0) return I8H_EINVAL;
  if (E > kMaxExperts || topk > kMaxTopk || topk > E) return I8H_EUNSUPPORTED;
  if ((int64_t)T * topk >= (int64_t)1 << 31) return I8H_EUNSUPPORTED;
  if (i8h::route_chunks(T, topk) * E >= (int64_t)1 << 31) return I8H_EUNSUPPORTED;
  if (T == 0) return I8H_OK;
  if (i8h::route_workspace_bytes(T, E, topk) > i8h::kRouteScratchBytes) return I8H_EUNSUPPORTED;
  if (!logits || !topk_ids || !topk_w || !expert_off || !sorted_pairs || !pair_pos) return I8H_EINVAL;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(expert_off, 4) ||
      !aligned(sorted_pairs, 4) || !aligned(pair_pos, 4))
    return I8H_EINVAL;
  void* ws = nullptr;
  if (i8h::route_scratch(as_stream(stream), &ws) != hipSuccess) return I8H_EHIP;
  return from_hip(i8h::launch_route(logits, T, E, topk, topk_ids, topk_w, expert_off, sorted_pairs, pair_pos, ws,
                                    nullptr, nullptr, 0, as_stream(stream)));
}

int hadamard128_rotate(const uint16_t* x, int64_t ldx, uint16_t* y, int64_t ldy, int T, int K, void* stream) {
  if (T < 0 || K <= 0 || (K % 128) != 0) return I8H_EINVAL;
  if (ldx < K || ldy < K || (ldx % 8) != 0 || (ldy % 8) != 0) return I8H_EINVAL;
  if (T == 0) return I8H_OK;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return I8H_EINVAL;
  if (x != y) {
    // other overlap would let one block read what another already wrote
    uintptr_t xb = reinterpret_cast<uintptr_t>(x), yb = reinterpret_cast<uintptr_t>(y);
    uintptr_t xe = xb + 2 * (uintptr_t)((int64_t)(T - 1) * ldx + K);
    uintptr_t ye = yb + 2 * (uintptr_t)((int64_t)(T - 1) * ldy + K);
    if (xb < ye && yb < xe) return I8H_EINVAL;
  } else if (ldx != ldy) {
    return I8H_EINVAL;
  }
  return from_hip(i8h::launch_fwht128(x, ldx, y, ldy, T, K, as_stream(stream)));
}

int moe_gateup_i8h_grouped(const uint16_t* x_rot, int T, int K, const int8_t* codes, const uint16_t* scales, int E,
                           int N, int topk, const int32_t* expert_off, const int32_t* sorted_pairs,
                           float* gate_up, float* act, void* stream) {
  return gateup_i8h(x_rot, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs, gate_up, act, false,
                    I8H_PATH_AUTO, stream);
}

int moe_gateup_i8h_grouped_path(const uint16_t* x_rot, int T, int K, const int8_t* codes, const uint16_t* scales,
                                int E, int N, int topk, const int32_t* expert_off, const int32_t* sorted_pairs,
                                float* gate_up, float* act, int path, void* stream) {
  return gateup_i8h(x_rot, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs, gate_up, act, false, path,
                    stream);
}

int moe_gateup_i8h_grouped_act_bf16(const uint16_t* x_rot, int T, int K, const int8_t* codes,
                                    const uint16_t* scales, int E, int N, int topk, const int32_t* expert_off,
                                    const int32_t* sorted_pairs, float* gate_up, uint16_t* act_bf16, int path,
                                    void* stream) {
  return gateup_i8h(x_rot, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs, gate_up, act_bf16, true,
                    path, stream);
}

int fp8_quantize_activations(const uint16_t* x, int T, int K, uint8_t* qx, float* sx, void* stream) {
  if (T < 0 || K <= 0 || (K % 128) != 0) return I8H_EINVAL;
  if (T == 0) return I8H_OK;
  if (!x || !qx || !sx || !aligned(x, 16) || !aligned(qx, 16) || !aligned(sx, 4)) return I8H_EINVAL;
  return from_hip(i8h::launch_fp8_act_quant(x, T, K, qx, sx, nullptr, as_stream(stream)));
}

size_t moe_gateup_fp8blk_workspace_size(int T, int K) {
  if (T <= 0 || K <= 0 || (K % 128) != 0) return 0;
  return Fp8Ws(T, K).total;
}

size_t moe_gateup_i8h_fused_workspace_size(int T, int K) {
  if (T <= 0 || K <= 0 || (K % 128) != 0) return 0;
  return auto_gemv(T, K) ? 0 : round_up((size_t)T * K * 2, 256);
}

int moe_gateup_i8h_grouped_fused(const uint16_t* x, int T, int K, const int8_t* codes, const uint16_t* scales, int E,
                                 int N, int topk, const int32_t* expert_off, const int32_t* sorted_pairs,
                                 float* gate_up, float* act, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  int rc = check_common_moe(T, K, E, N, topk);
  if (rc != I8H_OK) return rc;
  if ((N % 2) != 0) return I8H_EINVAL;                  // gate and up halves
  if ((N % 64) != 0) return I8H_EUNSUPPORTED;           // 32-row gate and up tiles
  if (T == 0) return I8H_OK;
  if (!x || !codes || !scales || !expert_off || !sorted_pairs) return I8H_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return I8H_EINVAL;
  if (!aligned(expert_off, 4) || !aligned(sorted_pairs, 4)) return I8H_EINVAL;
  if ((gate_up && !aligned(gate_up, 4)) || (act && !aligned(act, 4))) return I8H_EINVAL;
  size_t need = moe_gateup_i8h_fused_workspace_size(T, K);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return I8H_EINVAL;
  if (!gate_up && !act) return I8H_OK;
  hipStream_t st = as_stream(stream);
  if (auto_gemv(T, K))
    return from_hip(i8h::launch_gateup_i8h_gemv_rot(x, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs,
                                                    gate_up, act, st));
  uint16_t* xr = static_cast<uint16_t*>(workspace);
  if (i8h::launch_fwht128(x, K, xr, K, T, K, st) != hipSuccess) return I8H_EHIP;
  if (auto_path(T, K, E, N, topk) == I8H_PATH_TALL)
    return from_hip(i8h::launch_gateup_i8h_gemm_tall(xr, T, K, codes, scales, E, N, topk, expert_off,
                                                      sorted_pairs, gate_up, act, false, st));
  return from_hip(i8h::launch_gateup_i8h_skinny(xr, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs,
                                                gate_up, act, false, st));
}

int moe_route_gateup_i8h_decode(const float* logits, const uint16_t* x, int T, int K, const int8_t* codes,
                                const uint16_t* scales, int E, int N, int topk, int32_t* topk_ids, float* topk_w,
                                int32_t* expert_off, int32_t* sorted_pairs, int32_t* pair_pos, float* gate_up,
                                float* act, void* stream) {
  int rc = check_common_moe(T, K, E, N, topk);
  if (rc != I8H_OK) return rc;
  if ((N % 2) != 0) return I8H_EINVAL;                  // gate and up halves
  if ((N % 64) != 0) return I8H_EUNSUPPORTED;           // 32-row gate and up tiles
  if ((int64_t)T * topk > kDecodeMaxPairs || E > kDecodeMaxExperts || K > kGemvMaxK) return I8H_EUNSUPPORTED;
  if (T == 0) return I8H_OK;
  if (!logits || !x || !codes || !scales || !topk_ids || !topk_w || !expert_off || !sorted_pairs || !pair_pos)
    return I8H_EINVAL;
  if (!gate_up && !act) return I8H_EINVAL;
  if (!aligned(logits, 4) || !aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return I8H_EINVAL;
  if (!aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(expert_off, 4) || !aligned(sorted_pairs, 4) ||
      !aligned(pair_pos, 4))
    return I8H_EINVAL;
  if ((gate_up && !aligned(gate_up, 4)) || (act && !aligned(act, 4))) return I8H_EINVAL;
  return from_hip(i8h::launch_route_gateup_decode(logits, x, T, K, codes, scales, E, N, topk, topk_ids, topk_w,
                                                  expert_off, sorted_pairs, pair_pos, gate_up, act,
                                                  as_stream(stream)));
}

}  // extern "C"

namespace {

// act: float32 [P, I], or bf16 [P, I] when act_bf16
int gateup_fp8(const uint16_t* x, int T, int K, const uint8_t* codes, const uint16_t* scales, int E, int N,
               int topk, const int32_t* expert_off, const int32_t* sorted_pairs, float* gate_up, void* act,
               bool act_bf16, void* workspace, size_t workspace_bytes, int path, void* stream) {
  int rc = check_common_moe(T, K, E, N, topk);
  if (rc != I8H_OK) return rc;
  if ((N % 128) != 0) return I8H_EINVAL;
  if (path < I8H_PATH_AUTO || path > I8H_PATH_SKINNY) return I8H_EINVAL;
  if (path == I8H_PATH_GEMV || path == I8H_PATH_TALL) return I8H_EUNSUPPORTED;
  if (T == 0) return I8H_OK;
  if (!x || !codes || !scales || !expert_off || !sorted_pairs) return I8H_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(expert_off, 4) ||
      !aligned(sorted_pairs, 4))
    return I8H_EINVAL;
  if ((gate_up && !aligned(gate_up, 4)) || (act && !aligned(act, act_bf16 ? 2 : 4))) return I8H_EINVAL;
  size_t need = moe_gateup_fp8blk_workspace_size(T, K);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return I8H_EINVAL;
  if (!gate_up && !act) return I8H_OK;
  // as for int8: 128-pair passes once experts average 32 pairs, below that
  // the small-unit kernel
  if (path == I8H_PATH_AUTO)
    path = (int64_t)T * topk >= (int64_t)32 * E ? I8H_PATH_GEMM : I8H_PATH_SKINNY;
  Fp8Ws lay(T, K);
  uint8_t* qx = static_cast<uint8_t*>(workspace);
  float* sx = reinterpret_cast<float*>(qx + lay.sx_off);
  uint16_t* xq = reinterpret_cast<uint16_t*>(qx + lay.xq_off);
  hipStream_t st = as_stream(stream);
  hipError_t e = i8h::launch_fp8_act_quant(x, T, K, qx, sx, xq, st);
  if (e != hipSuccess) return I8H_EHIP;
  if (path == I8H_PATH_SKINNY)
    return from_hip(i8h::launch_gateup_fp8_skinny(xq, sx, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs,
                                                  gate_up, act, act_bf16, st));
  return from_hip(i8h::launch_gateup_fp8(xq, sx, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs,
                                         gate_up, act, act_bf16, st));
}

}  // namespace

extern "C" {

int moe_gateup_fp8blk_grouped_path(const uint16_t* x, int T, int K, const uint8_t* codes, const uint16_t* scales,
                                   int E, int N, int topk, const int32_t* expert_off, const int32_t* sorted_pairs,
                                   float* gate_up, float* act, void* workspace, size_t workspace_bytes, int path,
                                   void* stream) {
  return gateup_fp8(x, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs, gate_up, act, false, workspace,
                    workspace_bytes, path, stream);
}

int moe_gateup_fp8blk_grouped_act_bf16(const uint16_t* x, int T, int K, const uint8_t* codes,
                                       const uint16_t* scales, int E, int N, int topk, const int32_t* expert_off,
                                       const int32_t* sorted_pairs, float* gate_up, uint16_t* act_bf16,
                                       void* workspace, size_t workspace_bytes, int path, void* stream) {
  return gateup_fp8(x, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs, gate_up, act_bf16, true,
                    workspace, workspace_bytes, path, stream);
}

int moe_gateup_fp8blk_grouped(const uint16_t* x, int T, int K, const uint8_t* codes, const uint16_t* scales, int E,
                              int N, int topk, const int32_t* expert_off, const int32_t* sorted_pairs,
                              float* gate_up, float* act, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return moe_gateup_fp8blk_grouped_path(x, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs, gate_up, act,
                                        workspace, workspace_bytes, I8H_PATH_AUTO, stream);
}

// W8A8 int8 g128
int i8_quantize_activations(const uint16_t* x, int T, int K, int8_t* qx, float* sx, void* stream) {
  if (T < 0 || K <= 0 || (K % 128) != 0) return I8H_EINVAL;
  if ((int64_t)T * K >= (int64_t)1 << 31) return I8H_EUNSUPPORTED;
  if (T == 0) return I8H_OK;
  if (!x || !qx || !sx || !aligned(x, 16) || !aligned(qx, 8) || !aligned(sx, 4)) return I8H_EINVAL;
  return from_hip(i8h::launch_i8_act_quant(x, T, K, qx, sx, as_stream(stream)));
}

size_t moe_gateup_i8g_workspace_size(int T, int K) {
  if (T <= 0 || K <= 0 || (K % 128) != 0) return 0;
  return i8g_ws_total(T, K);
}

}  // extern "C"

namespace {

// act: float32 [P, I], or bf16 [P, I] when act_bf16
int gateup_i8g(const uint16_t* x, int T, int K, const int8_t* codes, const uint16_t* scales, int E, int N,
               int topk, const int32_t* expert_off, const int32_t* sorted_pairs, float* gate_up, void* act,
               bool act_bf16, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common_moe(T, K, E, N, topk);
  if (rc != I8H_OK) return rc;
  if ((N % 2) != 0) return I8H_EINVAL;                  // gate and up halves
  if ((N % 64) != 0) return I8H_EUNSUPPORTED;           // 32-row gate and up tiles
  if ((int64_t)N * K >= (int64_t)1 << 31) return I8H_EUNSUPPORTED;   // one expert's codes, 32-bit offsets
  if (T == 0) return I8H_OK;
  if (!x || !codes || !scales || !expert_off || !sorted_pairs) return I8H_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(expert_off, 4) ||
      !aligned(sorted_pairs, 4))
    return I8H_EINVAL;
  if ((gate_up && !aligned(gate_up, 4)) || (act && !aligned(act, act_bf16 ? 2 : 4))) return I8H_EINVAL;
  if (!workspace || workspace_bytes < i8g_ws_total(T, K) || !aligned(workspace, 256)) return I8H_EINVAL;
  if (!gate_up && !act) return I8H_OK;
  int8_t* qx = static_cast<int8_t*>(workspace);
  float* sx = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + i8g_sx_off(T, K));
  hipStream_t st = as_stream(stream);
  if (i8h::launch_i8_act_quant(x, T, K, qx, sx, st) != hipSuccess) return I8H_EHIP;
  return from_hip(i8h::launch_gateup_i8g(qx, sx, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs, gate_up,
                                         act, act_bf16, st));
}

}  // namespace

extern "C" {

int moe_gateup_i8g_grouped(const uint16_t* x, int T, int K, const int8_t* codes, const uint16_t* scales, int E,
                           int N, int topk, const int32_t* expert_off, const int32_t* sorted_pairs, float* gate_up,
                           float* act, void* workspace, size_t workspace_bytes, void* stream) {
  return gateup_i8g(x, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs, gate_up, act, false, workspace,
                    workspace_bytes, stream);
}

int moe_gateup_i8g_grouped_act_bf16(const uint16_t* x, int T, int K, const int8_t* codes, const uint16_t* scales,
                                    int E, int N, int topk, const int32_t* expert_off, const int32_t* sorted_pairs,
                                    float* gate_up, uint16_t* act_bf16, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return gateup_i8g(x, T, K, codes, scales, E, N, topk, expert_off, sorted_pairs, gate_up, act_bf16, true,
                    workspace, workspace_bytes, stream);
}



// bf16 grouped down projection + weighted combine
size_t moe_down_bf16_workspace_size(int T, int I, int H, int topk) {
  if (T <= 0 || I <= 0 || H <= 0 || topk <= 0) return 0;
  return DownWs(T, I, H, topk).total;
}

int moe_down_bf16_combine(const float* act, int T, int I, const uint16_t* w_down, int E, int H, int topk,
                          const int32_t* topk_ids, const float* topk_w, const int32_t* expert_off,
                          const int32_t* pair_pos, float* out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return down_combine(act, false, T, I, w_down, E, H, topk, topk_ids, topk_w, expert_off, pair_pos, out, workspace,
                      workspace_bytes, I8H_DOWN_AUTO, stream);
}

int moe_down_bf16_combine_path(const float* act, int T, int I, const uint16_t* w_down, int E, int H, int topk,
                               const int32_t* topk_ids, const float* topk_w, const int32_t* expert_off,
                               const int32_t* pair_pos, float* out, void* workspace, size_t workspace_bytes,
                               int path, void* stream) {
  return down_combine(act, false, T, I, w_down, E, H, topk, topk_ids, topk_w, expert_off, pair_pos, out, workspace,
                      workspace_bytes, path, stream);
}

size_t moe_down_bf16_act_bf16_workspace_size(int T, int I, int H, int topk) {
  if (T <= 0 || I <= 0 || H <= 0 || topk <= 0) return 0;
  return DownWs(T, I, H, topk).y;
}

int moe_down_bf16_combine_act_bf16(const uint16_t* act_bf16, int T, int I, const uint16_t* w_down, int E, int H,
                                   int topk, const int32_t* topk_ids, const float* topk_w,
                                   const int32_t* expert_off, const int32_t* pair_pos, float* out,
                                   void* workspace, size_t workspace_bytes, int path, void* stream) {
  return down_combine(act_bf16, true, T, I, w_down, E, H, topk, topk_ids, topk_w, expert_off, pair_pos, out,
                      workspace, workspace_bytes, path, stream);
}

// dense int8 linear with f16 group scales (the drafter's linears)
int linear_i8f16(const uint16_t* x, int T, int K, const int8_t* codes, const uint16_t* scales, int N, float* y,
                 void* stream) {
  if (T < 0 || K <= 0 || (K % 128) != 0 || N <= 0 || (N % 16) != 0) return I8H_EINVAL;
  if ((int64_t)T * K >= (int64_t)1 << 31 || (int64_t)N * K >= ((int64_t)1 << 40)) return I8H_EUNSUPPORTED;
  if (T == 0) return I8H_OK;
  if (!x || !codes || !scales || !y) return I8H_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(y, 4)) return I8H_EINVAL;
  return from_hip(i8h::launch_linear_i8f16(x, T, K, codes, scales, N, y, as_stream(stream)));
}

}  // extern "C"
