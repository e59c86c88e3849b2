// Decode-shaped grouped int8 Hadamard-domain gate_up (few tokens per expert).
//
// Format (int8 card, model table row "Weights"): int8 codes -127..127 in the
// 128-wide Hadamard domain, one bf16 scale per row and 128 of K. For sorted
// row r of expert e and token t:
//   gu[r, n] = sum_g s[e, n, g] * sum_{kk in g} q[e, n, kk] * x_rot[t, kk]
//   act[r, i] = gelu_tanh(gu[r, i]) * gu[r, I + i]
//
// Work split: the grid's y index is the slot of a non-empty expert (found by
// scanning expert_off on the device), x covers row pairs (i, I + i); one wave
// owns one row pair. Lane l reads 16-byte pieces kk = 16 (l + 64 c) of both
// rows, so each wave load is 1 KB of contiguous codes. Codes become float
// exactly (sign-extended byte converts), products with the bf16 activations
// are exact in float32 FMAs, each 16-value partial is scaled by its group's
// bf16 scale, and a fixed-order wave reduction finishes the dot product. The
// codes of the row pair are read once and reused for every pair (token) of
// the expert.

#include "common.hpp"
#include "launch.hpp"

namespace i8h {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

// Expert owning the s-th non-empty run of expert_off (in expert order), or
// -1. Same answer in every lane.
__device__ __forceinline__ int nth_nonempty_expert(const int32_t* __restrict__ off, int E, int s, int lane) {
  int seen = 0;
  for (int base = 0; base < E; base += kWave) {
    int e = base + lane;
    bool ne = false;
    if (e < E) ne = off[e + 1] > off[e];
    uint64_t m = __ballot(ne);
    int c = __popcll(m);
    if (s < seen + c) {
      int want = s - seen;  // position of the wanted set bit
      for (int i = 0; i < want; ++i) m &= m - 1;
      return base + __ffsll((unsigned long long)m) - 1;
    }
    seen += c;
  }
  return -1;
}

template <int NCH>
__global__ void __launch_bounds__(kGemvThreads)
k_gateup_i8h_gemv(const uint16_t* __restrict__ xrot, int K, const int8_t* __restrict__ codes,
                  const uint16_t* __restrict__ scales, int E, int N, int k,
                  const int32_t* __restrict__ expert_off, const int32_t* __restrict__ sorted_pairs,
                  float* __restrict__ gu, float* __restrict__ act) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int I = N / 2;
  const int i = blockIdx.x * kGemvWaves + wave;
  if (i >= I) return;
  const int e = nth_nonempty_expert(expert_off, E, blockIdx.y, lane);
  if (e < 0) return;
  const int r0 = expert_off[e], r1 = expert_off[e + 1];
  const int G = K / kGroup;

  const int8_t* rowg = codes + ((size_t)e * N + i) * K;
  const int8_t* rowu = codes + ((size_t)e * N + I + i) * K;
  const uint16_t* sg = scales + ((size_t)e * N + i) * G;
  const uint16_t* su = scales + ((size_t)e * N + I + i) * G;

  // codes of both rows: NCH pieces of 16 bytes per lane
  u32x4 cg[NCH], cu[NCH];
  float scg[NCH], scu[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    int kk = 16 * (lane + kWave * c);
    if (kk < K) {
      cg[c] = *reinterpret_cast<const u32x4*>(rowg + kk);
      cu[c] = *reinterpret_cast<const u32x4*>(rowu + kk);
      scg[c] = bf16_to_f32(sg[kk / kGroup]);
      scu[c] = bf16_to_f32(su[kk / kGroup]);
    } else {
      cg[c] = u32x4{0u, 0u, 0u, 0u};
      cu[c] = u32x4{0u, 0u, 0u, 0u};
      scg[c] = 0.0f;
      scu[c] = 0.0f;
    }
  }
  for (int r = r0; r < r1; ++r) {
    const int t = sorted_pairs[r] / k;
    const uint16_t* xr = xrot + (size_t)t * K;
    float accg = 0.0f, accu = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      int kk = 16 * (lane + kWave * c);
      u32x4 xa = {0u, 0u, 0u, 0u}, xb = {0u, 0u, 0u, 0u};
      if (kk < K) {
        xa = *reinterpret_cast<const u32x4*>(xr + kk);
        xb = *reinterpret_cast<const u32x4*>(xr + kk + 8);
      }
      // x[kk + j] for j = 0..15, and the codes at the same positions
      float xv[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        xv[2 * w] = bf16_lo(xa[w]);
        xv[2 * w + 1] = bf16_hi(xa[w]);
        xv[8 + 2 * w] = bf16_lo(xb[w]);
        xv[8 + 2 * w + 1] = bf16_hi(xb[w]);
      }
      float pg0 = 0.0f, pg1 = 0.0f, pu0 = 0.0f, pu1 = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pg0 = fmaf(sbyte<0>(cg[c][w]), xv[4 * w + 0], pg0);
        pg1 = fmaf(sbyte<1>(cg[c][w]), xv[4 * w + 1], pg1);
        pg0 = fmaf(sbyte<2>(cg[c][w]), xv[4 * w + 2], pg0);
        pg1 = fmaf(sbyte<3>(cg[c][w]), xv[4 * w + 3], pg1);
        pu0 = fmaf(sbyte<0>(cu[c][w]), xv[4 * w + 0], pu0);
        pu1 = fmaf(sbyte<1>(cu[c][w]), xv[4 * w + 1], pu1);
        pu0 = fmaf(sbyte<2>(cu[c][w]), xv[4 * w + 2], pu0);
        pu1 = fmaf(sbyte<3>(cu[c][w]), xv[4 * w + 3], pu1);
      }
      accg = fmaf(scg[c], pg0 + pg1, accg);
      accu = fmaf(scu[c], pu0 + pu1, accu);
    }
    float g = wave_sum(accg);
    float u = wave_sum(accu);
    if (lane == 0) {
      if (gu) {
        gu[(size_t)r * N + i] = g;
        gu[(size_t)r * N + I + i] = u;
      }
      if (act) act[(size_t)r * I + i] = gelu_tanh(g) * u;
    }
  }
}

hipError_t launch_gateup_i8h_gemv(const uint16_t* xrot, int T, int K, const int8_t* codes,
                                  const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                  const int32_t* sorted_pairs, float* gu, float* act, hipStream_t st) {
  int P = T * k;
  int slots = P < E ? P : E;  // at most this many experts can be non-empty
  int I = N / 2;
  dim3 grid(cdiv(I, kGemvWaves), slots);
  int nch = cdiv(K, 16 * kWave);
  if (nch <= 1)
    k_gateup_i8h_gemv<1><<<grid, kGemvThreads, 0, st>>>(xrot, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu, act);
  else if (nch <= 2)
    k_gateup_i8h_gemv<2><<<grid, kGemvThreads, 0, st>>>(xrot, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu, act);
  else if (nch <= 4)
    k_gateup_i8h_gemv<4><<<grid, kGemvThreads, 0, st>>>(xrot, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu, act);
  else
    k_gateup_i8h_gemv<8><<<grid, kGemvThreads, 0, st>>>(xrot, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu, act);
  return hipGetLastError();
}

}  // namespace i8h
