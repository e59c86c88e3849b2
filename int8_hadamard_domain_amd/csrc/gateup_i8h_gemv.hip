// Decode-shaped grouped int8 Hadamard-domain gate_up (few tokens per expert).
//
// Format (int8 card, model table row "Weights"): int8 codes -127..127 in the
// 128-wide Hadamard domain, one bf16 scale per row and 128 of K. For sorted
// row r of expert e and token t:
//   gu[r, n] = sum_g s[e, n, g] * sum_{kk in g} q[e, n, kk] * x_rot[t, kk]
//   act[r, i] = gelu_tanh(gu[r, i]) * gu[r, I + i]
//
// Work split: grid y = slot of a non-empty expert (found by scanning
// expert_off on the device), grid x = groups of row pairs (i, I + i). Each
// wave owns RPW row pairs and issues all of their code loads at once (lane l
// reads the 16-byte pieces kk = 16 (l + 64 c) of every row: each wave load is
// 1 KB of one row), so many kilobytes are in flight per wave. Codes become
// float exactly (sign-extended byte converts), products with the bf16
// activations are exact in float32 FMAs, each 16-value partial is scaled by
// its group's bf16 scale, and one transposing reduction (xor 32, 16, 8 keep
// half of the values each step; then xor 4, 2, 1) finishes all 2*RPW dot
// products of the wave in a fixed order. The codes are read once and reused
// for every token routed to the expert.
//
// ROT = true takes unrotated activations and applies the 128-wide Hadamard
// rotation in the prologue: the 8 lanes holding one 128-block run four
// butterfly stages in registers and three across lanes (xor 1, 2, 4), scale
// by 1/sqrt(128) and round to bf16, exactly the activation the separate
// rotation call would produce up to float32 rounding order.

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

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

// One transposing step at lane distance M over NV values: the lane with bit
// M clear keeps the first half (adding its partner's first half), the other
// keeps the second half.
template <int M, int NV>
__device__ __forceinline__ void fold_half(float (&v)[NV], int lane) {
  const bool hi = (lane & M) != 0;
#pragma unroll
  for (int q = 0; q < NV / 2; ++q) {
    float send = hi ? v[q] : v[NV / 2 + q];
    float keep = hi ? v[NV / 2 + q] : v[q];
    v[q] = keep + xor_lane<M>(send);
  }
}

// 16 consecutive values of a 128-block held by lane (lane % 8) of its
// 8-lane group -> rotated, rounded to bf16, back in float.
__device__ __forceinline__ void rotate16(float (&xv)[16], int lane) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        float a = xv[i], b = xv[i + h];
        xv[i] = a + b;
        xv[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = hadamard_xlane<1>(xv[i], lane);
    v = hadamard_xlane<2>(v, lane);
    v = hadamard_xlane<4>(v, lane);
    const float rs = 0.08838834764831845f;  // 1/sqrt(128)
    xv[i] = (float)(__bf16)(v * rs);
  }
}

template <int NCH, int RPW, bool ROT>
__global__ void __launch_bounds__(kGemvThreads)
k_gateup_i8h_gemv(const uint16_t* __restrict__ xin, int K, const int8_t* __restrict__ codes,
                  const uint16_t* __restrict__ scales, int E, int N, int k,
                  const int32_t* __restrict__ expert_off, const int32_t* __restrict__ sorted_pairs,
                  float* __restrict__ gu, float* __restrict__ act) {
  static_assert(RPW == 2 || RPW == 4, "2*RPW values per lane are folded over bits 5..");
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int I = N / 2;
  const int i0 = (blockIdx.x * kGemvWaves + wave) * RPW;  // I % RPW == 0, so all RPW rows exist
  if (i0 >= I) return;
  const int e = nth_nonempty_expert(expert_off, E, blockIdx.y, lane);
  if (e < 0) return;
  const int r0 = expert_off[e], r1 = expert_off[e + 1];
  const int G = K / kGroup;

  u32x4 cg[RPW][NCH], cu[RPW][NCH];
  float sg[RPW][NCH], su[RPW][NCH];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int8_t* rowg = codes + ((size_t)e * N + i0 + j) * K;
    const int8_t* rowu = codes + ((size_t)e * N + I + i0 + j) * K;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      int kk = 16 * (lane + kWave * c);
      if (kk < K) {
        cg[j][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowg + kk));
        cu[j][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowu + kk));
      } else {
        cg[j][c] = u32x4{0u, 0u, 0u, 0u};
        cu[j][c] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const uint16_t* srg = scales + ((size_t)e * N + i0 + j) * G;
    const uint16_t* sru = scales + ((size_t)e * N + I + i0 + j) * G;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      int kk = 16 * (lane + kWave * c);
      int g = kk < K ? kk / kGroup : 0;
      sg[j][c] = bf16_to_f32(srg[g]);
      su[j][c] = bf16_to_f32(sru[g]);
    }
  }

  for (int r = r0; r < r1; ++r) {
    const int t = sorted_pairs[r] / k;
    const uint16_t* xr = xin + (size_t)t * K;
    float v[2 * RPW];
#pragma unroll
    for (int q = 0; q < 2 * RPW; ++q) v[q] = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      int kk = 16 * (lane + kWave * c);
      u32x4 xa = {0u, 0u, 0u, 0u}, xb = {0u, 0u, 0u, 0u};
      if (kk < K) {
        xa = *reinterpret_cast<const u32x4*>(xr + kk);
        xb = *reinterpret_cast<const u32x4*>(xr + kk + 8);
      }
      float xv[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        xv[2 * w] = bf16_lo(xa[w]);
        xv[2 * w + 1] = bf16_hi(xa[w]);
        xv[8 + 2 * w] = bf16_lo(xb[w]);
        xv[8 + 2 * w + 1] = bf16_hi(xb[w]);
      }
      if constexpr (ROT) rotate16(xv, lane);
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        // the codes are loop-invariant; an empty asm keeps their conversion
        // inside the loop (hoisted, it would hold every code as a float)
        u32x4 qg = cg[j][c], qu = cu[j][c];
        asm volatile("" : "+v"(qg), "+v"(qu));
        float pg0 = 0.0f, pg1 = 0.0f, pu0 = 0.0f, pu1 = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pg0 = fmaf(sbyte<0>(qg[w]), xv[4 * w + 0], pg0);
          pg1 = fmaf(sbyte<1>(qg[w]), xv[4 * w + 1], pg1);
          pg0 = fmaf(sbyte<2>(qg[w]), xv[4 * w + 2], pg0);
          pg1 = fmaf(sbyte<3>(qg[w]), xv[4 * w + 3], pg1);
          pu0 = fmaf(sbyte<0>(qu[w]), xv[4 * w + 0], pu0);
          pu1 = fmaf(sbyte<1>(qu[w]), xv[4 * w + 1], pu1);
          pu0 = fmaf(sbyte<2>(qu[w]), xv[4 * w + 2], pu0);
          pu1 = fmaf(sbyte<3>(qu[w]), xv[4 * w + 3], pu1);
        }
        v[2 * j] = fmaf(sg[j][c], pg0 + pg1, v[2 * j]);
        v[2 * j + 1] = fmaf(su[j][c], pu0 + pu1, v[2 * j + 1]);
      }
    }
    // v = (g0, u0, g1, u1, ...): fold halves over bits 5, 4 (and 3), then sum
    // the lanes that share the kept index
    fold_half<32>(v, lane);            // v[0 .. RPW) now hold the kept half
    float w[RPW];
#pragma unroll
    for (int q = 0; q < RPW; ++q) w[q] = v[q];
    fold_half<16>(w, lane);            // w[0 .. RPW/2)
    float s;
    int up_bit;
    if constexpr (RPW == 4) {
      float z[2] = {w[0], w[1]};
      fold_half<8>(z, lane);
      s = z[0];
      s += xor_lane<1>(s);
      s += xor_lane<2>(s);
      s += xor_lane<4>(s);
      up_bit = 8;
    } else {
      s = w[0];
      s += xor_lane<1>(s);
      s += xor_lane<2>(s);
      s += xor_lane<4>(s);
      s += xor_lane<8>(s);
      up_bit = 16;
    }
    // lane holds gate (up_bit clear) or up (up_bit set) of pair j
    float other = (up_bit == 8) ? xor_lane<8>(s) : xor_lane<16>(s);
    const int jmask = (up_bit == 8) ? 15 : 31;
    if ((lane & jmask) == 0) {
      const int j = (up_bit == 8) ? (lane >> 4) : (lane >> 5);
      const float g = s, u = other;
      if (gu) {
        gu[(size_t)r * N + i0 + j] = g;
        gu[(size_t)r * N + I + i0 + j] = u;
      }
      if (act) act[(size_t)r * I + i0 + j] = gelu_tanh(g) * u;
    }
  }
}

template <bool ROT>
static hipError_t launch_gemv(const uint16_t* x, int T, int K, const int8_t* codes, const uint16_t* scales, int E,
                              int N, int k, const int32_t* expert_off, const int32_t* sorted_pairs, float* gu,
                              float* act, hipStream_t st) {
  int P = T * k;
  int slots = P < E ? P : E;  // at most this many experts can be non-empty
  int I = N / 2;
  int nch = cdiv(K, 16 * kWave);
  if (nch <= 1) {
    dim3 grid(cdiv(I, kGemvWaves * 4), slots);
    k_gateup_i8h_gemv<1, 4, ROT><<<grid, kGemvThreads, 0, st>>>(x, K, codes, scales, E, N, k, expert_off,
                                                                sorted_pairs, gu, act);
  } else if (nch <= 2) {
    dim3 grid(cdiv(I, kGemvWaves * 4), slots);
    k_gateup_i8h_gemv<2, 4, ROT><<<grid, kGemvThreads, 0, st>>>(x, K, codes, scales, E, N, k, expert_off,
                                                                sorted_pairs, gu, act);
  } else {
    dim3 grid(cdiv(I, kGemvWaves * 2), slots);
    k_gateup_i8h_gemv<4, 2, ROT><<<grid, kGemvThreads, 0, st>>>(x, K, codes, scales, E, N, k, expert_off,
                                                                sorted_pairs, gu, act);
  }
  return hipGetLastError();
}

hipError_t launch_gateup_i8h_gemv(const uint16_t* xrot, int T, int K, const int8_t* codes,
                                  const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                  const int32_t* sorted_pairs, float* gu, float* act, hipStream_t st) {
  return launch_gemv<false>(xrot, T, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu, act, st);
}

hipError_t launch_gateup_i8h_gemv_rot(const uint16_t* x, int T, int K, const int8_t* codes,
                                      const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                      const int32_t* sorted_pairs, float* gu, float* act, hipStream_t st) {
  return launch_gemv<true>(x, T, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu, act, st);
}

}  // namespace i8h
