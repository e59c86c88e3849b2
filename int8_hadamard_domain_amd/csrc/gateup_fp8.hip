// FP8 E4M3 128x128-block grouped gate_up on gfx950's FP8 MFMA.
//
// Weights (FP8 card, model table row "Weights"): E4M3 codes per 128x128 block
// with one bf16 scale per block. The activations are bf16; FP8 MFMA needs
// FP8 operands, so they are quantized per token and per 128 of K with a
// float32 scale (the granularity of the int8 12B card's activations, header
// table row "Format"):
//   sx[t, g] = float32(amax / 448), qx = E4M3(x / sx) nearest even, saturating.
// Then
//   gu[r, n] = sum_g (sw[e, n/128, g] * sx[t, g]) * sum_{kk in g} qw * qx
//   act[r, i] = gelu_tanh(gu[r, i]) * gu[r, I + i].
//
// The E4M3 encoder is written out here (bit-exact, independent of the
// hardware convert's rounding and clamping modes): round the float32 to 3
// significand bits with ties to even, subnormals below 2^-6 in steps of 2^-9,
// magnitudes above 448 saturate, the sign bit is kept.
//
// GEMM: same unit and wave split as the int8 kernel. v_mfma_f32_32x32x64
// (f8f6f4 with both operands E4M3) takes 32 codes per lane for row/column
// l % 32 from k-half l / 32; two instructions cover a 128-K group. Element
// j of a lane in step s, half h stands for kk = 128 g + 64 h + 32 s + j for
// both operands. Each group's product is folded with the product of the
// block scale and the per-row activation scale.

#include "common.hpp"
#include "launch.hpp"

namespace i8h {

// ---- activation quantizer ------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_from_f32(float v) {
  uint32_t bits = __float_as_uint(v);
  uint32_t sign = (bits >> 24) & 0x80u;
  uint32_t mag = bits & 0x7fffffffu;
  float a = __uint_as_float(mag);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: steps of 2^-9
    code = (uint32_t)rintf(a * 512.0f);      // exact scaling, nearest even; 8 -> 0x08
  } else if (a > 448.0f) {
    code = 0x7eu;
  } else {
    uint32_t q = mag >> 20;                  // fp32 exponent and top 3 significand bits
    uint32_t rem = mag & 0xfffffu;
    uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (q & 1u));
    code = q + up - (120u << 3);             // rebias exponent 127 -> 7
    if (code > 0x7eu) code = 0x7eu;
  }
  return sign | code;
}

constexpr int kQuantThreads = 256;

// 16 lanes per 128-value group, 8 values per lane.
__global__ void __launch_bounds__(kQuantThreads)
k_fp8_act_quant(const uint16_t* __restrict__ x, int T, int K, uint8_t* __restrict__ qx, float* __restrict__ sx) {
  const int G = K / kGroup;
  int64_t grp = (int64_t)blockIdx.x * (kQuantThreads / 16) + threadIdx.x / 16;
  int j = threadIdx.x % 16;
  bool live = grp < (int64_t)T * G;
  int64_t t = live ? grp / G : 0;
  int g = live ? int(grp % G) : 0;
  u32x4 w = {0u, 0u, 0u, 0u};
  if (live) w = *reinterpret_cast<const u32x4*>(x + t * K + g * kGroup + 8 * j);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
  float s = amax / 448.0f;                   // IEEE single division
  uint32_t out0 = 0, out1 = 0;
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out0 |= e4m3_from_f32(v[i] / s) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) out1 |= e4m3_from_f32(v[4 + i] / s) << (8 * i);
  }
  if (live) {
    *reinterpret_cast<u32x2*>(qx + t * K + g * kGroup + 8 * j) = u32x2{out0, out1};
    if (j == 0) sx[t * G + g] = s;
  }
}

hipError_t launch_fp8_act_quant(const uint16_t* x, int T, int K, uint8_t* qx, float* sx, hipStream_t st) {
  int64_t groups = (int64_t)T * (K / kGroup);
  int per = kQuantThreads / 16;
  int grid = (int)((groups + per - 1) / per);
  k_fp8_act_quant<<<grid, kQuantThreads, 0, st>>>(x, T, K, qx, sx);
  return hipGetLastError();
}

// ---- grouped GEMM ----------------------------------------------------------
constexpr int kF8Threads = 256;
constexpr int kF8Waves = 4;
constexpr int kF8NTileGate = 32 * kF8Waves;
constexpr int kF8MT = 64;
constexpr int kF8MTiles = kF8MT / 32;
constexpr int kF8ARow = 144;  // bytes per LDS row: 128 codes + 16 pad

__global__ void __launch_bounds__(kF8Threads)
k_gateup_fp8_gemm(const uint8_t* __restrict__ qx, const float* __restrict__ sx, int K,
                  const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int E, int N, int k,
                  const int32_t* __restrict__ expert_off, const int32_t* __restrict__ sorted_pairs,
                  float* __restrict__ gu, float* __restrict__ act) {
  __shared__ __attribute__((aligned(16))) uint8_t As[kF8MT * kF8ARow];
  __shared__ float Ss[kF8MT];
  const int e = blockIdx.y;
  const int r0 = expert_off[e];
  const int m_e = expert_off[e + 1] - r0;
  if (m_e <= 0) return;
  const int I = N / 2, G = K / kGroup, NB = N / kGroup;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane % 32, half = lane / 32;
  const int i0 = blockIdx.x * kF8NTileGate + 32 * wave;
  const bool live = i0 < I;
  const int ng = i0 + col, nu = I + i0 + col;
  const uint8_t* cgp = codes + ((size_t)e * N + (live ? ng : 0)) * K + 64 * half;
  const uint8_t* cup = codes + ((size_t)e * N + (live ? nu : 0)) * K + 64 * half;
  // the wave's 32 gate rows share one 128-row scale block, as do its up rows
  const uint16_t* swg = scales + ((size_t)e * NB + (live ? i0 / kGroup : 0)) * G;
  const uint16_t* swu = scales + ((size_t)e * NB + (live ? (I + i0) / kGroup : 0)) * G;

  for (int mb = 0; mb < m_e; mb += kF8MT) {
    const int rows = min(kF8MT, m_e - mb);
    constexpr int kPieces = kF8MT * 8 / kF8Threads;  // 16-byte pieces per thread
    int tok[kPieces];
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      int row = (tid + kF8Threads * q) / 8;
      tok[q] = row < rows ? sorted_pairs[r0 + mb + row] / k : -1;
    }
    int stok = tid < rows ? sorted_pairs[r0 + mb + tid] / k : -1;
    f32x16 acc[kF8MTiles][2];
#pragma unroll
    for (int a = 0; a < kF8MTiles; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.0f;

    for (int g = 0; g < G; ++g) {
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kPieces; ++q) {
        int p = tid + kF8Threads * q;
        int row = p / 8, c = p % 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (tok[q] >= 0) v = *reinterpret_cast<const u32x4*>(qx + (size_t)tok[q] * K + g * kGroup + 16 * c);
        *reinterpret_cast<u32x4*>(&As[row * kF8ARow + 16 * c]) = v;
      }
      if (tid < kF8MT) Ss[tid] = stok >= 0 ? sx[(size_t)stok * G + g] : 0.0f;
      __syncthreads();
      if (!live) continue;
      u32x4 cg[4], cu[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        cg[j] = *reinterpret_cast<const u32x4*>(cgp + (size_t)g * kGroup + 16 * j);
        cu[j] = *reinterpret_cast<const u32x4*>(cup + (size_t)g * kGroup + 16 * j);
      }
      f32x16 tmp[kF8MTiles][2];
#pragma unroll
      for (int a = 0; a < kF8MTiles; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int j = 0; j < 16; ++j) tmp[a][b][j] = 0.0f;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        i32x8 bg, bu;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          bg[d] = (int)cg[2 * s][d];
          bg[4 + d] = (int)cg[2 * s + 1][d];
          bu[d] = (int)cu[2 * s][d];
          bu[4 + d] = (int)cu[2 * s + 1][d];
        }
#pragma unroll
        for (int a = 0; a < kF8MTiles; ++a) {
          if (a * 32 < rows) {
            const uint8_t* ap = &As[(a * 32 + col) * kF8ARow + 64 * half + 32 * s];
            u32x4 lo = *reinterpret_cast<const u32x4*>(ap);
            u32x4 hi = *reinterpret_cast<const u32x4*>(ap + 16);
            i32x8 av;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              av[d] = (int)lo[d];
              av[4 + d] = (int)hi[d];
            }
            tmp[a][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bg, tmp[a][0], 0, 0, 0, 0, 0, 0);
            tmp[a][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bu, tmp[a][1], 0, 0, 0, 0, 0, 0);
          }
        }
      }
      const float wg = bf16_to_f32(swg[g]), wu = bf16_to_f32(swu[g]);
#pragma unroll
      for (int a = 0; a < kF8MTiles; ++a) {
        if (a * 32 < rows) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            float s_m = Ss[a * 32 + 8 * (j / 4) + 4 * half + (j % 4)];
            acc[a][0][j] = fmaf(tmp[a][0][j], wg * s_m, acc[a][0][j]);
            acc[a][1][j] = fmaf(tmp[a][1][j], wu * s_m, acc[a][1][j]);
          }
        }
      }
    }
    if (live) {
#pragma unroll
      for (int a = 0; a < kF8MTiles; ++a) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          int m = a * 32 + 8 * (j / 4) + 4 * half + (j % 4);
          if (m < rows) {
            size_t r = (size_t)(r0 + mb + m);
            float gv = acc[a][0][j], uv = acc[a][1][j];
            if (gu) {
              gu[r * N + ng] = gv;
              gu[r * N + nu] = uv;
            }
            if (act) act[r * I + i0 + col] = gelu_tanh(gv) * uv;
          }
        }
      }
    }
  }
}

hipError_t launch_gateup_fp8(const uint8_t* qx, const float* sx, int T, int K, const uint8_t* codes,
                             const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                             const int32_t* sorted_pairs, float* gu, float* act, hipStream_t st) {
  (void)T;
  int I = N / 2;
  dim3 grid(cdiv(I, kF8NTileGate), E);
  k_gateup_fp8_gemm<<<grid, kF8Threads, 0, st>>>(qx, sx, K, codes, scales, E, N, k, expert_off, sorted_pairs,
                                                 gu, act);
  return hipGetLastError();
}

}  // namespace i8h
