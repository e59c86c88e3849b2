// Verify/prefill-shaped grouped int8 Hadamard-domain gate_up on bf16 MFMA.
//
// Format (int8 card, model table row "Weights"): int8 codes -127..127 in the
// 128-wide Hadamard domain, one bf16 scale per row and 128 of K:
//   gu[r, n]  = sum_g s[e, n, g] * sum_{kk in g} q[e, n, kk] * x_rot[t, kk]
//   act[r, i] = gelu_tanh(gu[r, i]) * gu[r, I + i]
//
// Work unit = (expert e, tile of 128 gate rows + the 128 matching up rows).
// Every unit walks all pairs of its expert (m-passes of kMT rows), so each
// code byte is read from HBM once per pass. Four waves split the unit's
// rows: wave w owns gate rows i0..i0+31 and up rows I+i0..I+i0+31, so the
// gate and up values of one output meet in the same lane (fused epilogue).
//
// Per 128-K group: the activation rows of the pass (gathered by sorted pair)
// are staged in LDS as bf16; each lane loads its B fragments (8 codes of one
// row per MFMA) straight from global memory and converts them to bf16
// exactly (|q| <= 127 fits bf16's 8-bit significand). v_mfma_f32_32x32x16_bf16
// accumulates the group into a temporary tile that is then folded into the
// float32 result with the group's scale: main += tmp * s[n, g]. (Scaling the
// codes first would round each weight to bf16.)
//
// MFMA operand mapping. For 32x32x16 bf16, lane l supplies 8 values for row
// (A) or column (B) l % 32 from k-half l / 32, and element j of A meets
// element j of B. The contraction is order-free, so the K positions a lane
// feeds are chosen for contiguous loads: in group g, step s, half h, element
// j stands for kk = 128 g + 64 h + 8 s + j, the same for A and B. The 32x32
// result sits in lane l as column l % 32, rows 8 (j / 4) + 4 (l / 32) + j % 4.

#include "common.hpp"
#include "launch.hpp"

namespace i8h {

constexpr int kGemmThreads = 256;
constexpr int kGemmWaves = 4;
constexpr int kNTileGate = 32 * kGemmWaves;  // gate rows per unit
constexpr int kMT = 64;                      // pairs per m-pass
constexpr int kMTiles = kMT / 32;
constexpr int kARowPad = 136;                // bf16 per LDS row (128 + 8 pad)

__device__ __forceinline__ bf16x8 codes8_to_bf16(uint32_t lo, uint32_t hi) {
  u32x4 p;
  p[0] = pack_bf16x2(sbyte<0>(lo), sbyte<1>(lo));
  p[1] = pack_bf16x2(sbyte<2>(lo), sbyte<3>(lo));
  p[2] = pack_bf16x2(sbyte<0>(hi), sbyte<1>(hi));
  p[3] = pack_bf16x2(sbyte<2>(hi), sbyte<3>(hi));
  return __builtin_bit_cast(bf16x8, p);
}

__global__ void __launch_bounds__(kGemmThreads)
k_gateup_i8h_gemm(const uint16_t* __restrict__ xrot, int K, const int8_t* __restrict__ codes,
                  const uint16_t* __restrict__ scales, int E, int N, int k,
                  const int32_t* __restrict__ expert_off, const int32_t* __restrict__ sorted_pairs,
                  float* __restrict__ gu, float* __restrict__ act) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kMT * kARowPad];
  const int e = blockIdx.y;
  const int r0 = expert_off[e];
  const int m_e = expert_off[e + 1] - r0;
  if (m_e <= 0) return;
  const int I = N / 2, G = K / kGroup;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane % 32, half = lane / 32;
  const int i0 = blockIdx.x * kNTileGate + 32 * wave;
  const bool live = i0 < I;  // I is a multiple of 32: a live wave has 32 rows
  const int ng = i0 + col, nu = I + i0 + col;
  const int8_t* cgp = codes + ((size_t)e * N + (live ? ng : 0)) * K + 64 * half;
  const int8_t* cup = codes + ((size_t)e * N + (live ? nu : 0)) * K + 64 * half;
  const uint16_t* sgp = scales + ((size_t)e * N + (live ? ng : 0)) * G;
  const uint16_t* sup = scales + ((size_t)e * N + (live ? nu : 0)) * G;

  for (int mb = 0; mb < m_e; mb += kMT) {
    const int rows = min(kMT, m_e - mb);
    // tokens of the rows this thread stages: piece p = tid + 256 q -> row p / 16
    constexpr int kPieces = kMT * 16 / kGemmThreads;
    int tok[kPieces];
#pragma unroll
    for (int q = 0; q < kPieces; ++q) {
      int row = (tid + kGemmThreads * q) / 16;
      tok[q] = row < rows ? sorted_pairs[r0 + mb + row] / k : -1;
    }
    f32x16 acc[kMTiles][2];
#pragma unroll
    for (int a = 0; a < kMTiles; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.0f;

    for (int g = 0; g < G; ++g) {
      __syncthreads();  // the previous group's LDS reads are done
#pragma unroll
      for (int q = 0; q < kPieces; ++q) {
        int p = tid + kGemmThreads * q;
        int row = p / 16, c = p % 16;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (tok[q] >= 0) v = *reinterpret_cast<const u32x4*>(xrot + (size_t)tok[q] * K + g * kGroup + 8 * c);
        *reinterpret_cast<u32x4*>(&As[row * kARowPad + 8 * c]) = v;
      }
      __syncthreads();
      if (!live) continue;
      u32x4 cg[4], cu[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        cg[j] = *reinterpret_cast<const u32x4*>(cgp + (size_t)g * kGroup + 16 * j);
        cu[j] = *reinterpret_cast<const u32x4*>(cup + (size_t)g * kGroup + 16 * j);
      }
      f32x16 tmp[kMTiles][2];
#pragma unroll
      for (int a = 0; a < kMTiles; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int j = 0; j < 16; ++j) tmp[a][b][j] = 0.0f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bf16x8 bg = codes8_to_bf16(cg[s / 2][2 * (s % 2)], cg[s / 2][2 * (s % 2) + 1]);
        bf16x8 bu = codes8_to_bf16(cu[s / 2][2 * (s % 2)], cu[s / 2][2 * (s % 2) + 1]);
#pragma unroll
        for (int a = 0; a < kMTiles; ++a) {
          if (a * 32 < rows) {
            bf16x8 av = *reinterpret_cast<const bf16x8*>(&As[(a * 32 + col) * kARowPad + 64 * half + 8 * s]);
            tmp[a][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bg, tmp[a][0], 0, 0, 0);
            tmp[a][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bu, tmp[a][1], 0, 0, 0);
          }
        }
      }
      const float sg = bf16_to_f32(sgp[g]), su = bf16_to_f32(sup[g]);
#pragma unroll
      for (int a = 0; a < kMTiles; ++a) {
        if (a * 32 < rows) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            acc[a][0][j] = fmaf(tmp[a][0][j], sg, acc[a][0][j]);
            acc[a][1][j] = fmaf(tmp[a][1][j], su, acc[a][1][j]);
          }
        }
      }
    }
    if (live) {
#pragma unroll
      for (int a = 0; a < kMTiles; ++a) {
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

hipError_t launch_gateup_i8h_gemm(const uint16_t* xrot, int T, int K, const int8_t* codes,
                                  const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                  const int32_t* sorted_pairs, float* gu, float* act, hipStream_t st) {
  (void)T;
  int I = N / 2;
  dim3 grid(cdiv(I, kNTileGate), E);
  k_gateup_i8h_gemm<<<grid, kGemmThreads, 0, st>>>(xrot, K, codes, scales, E, N, k, expert_off, sorted_pairs,
                                                   gu, act);
  return hipGetLastError();
}

}  // namespace i8h
