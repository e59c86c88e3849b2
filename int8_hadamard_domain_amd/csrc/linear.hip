// Dense int8 linear with an f16 scale per row and 128 of K, no transform: the
// DFlash drafter's linears of the int8 card (model table, row "Speculator";
// recipe lines `rtn codes=i8 group=128 scale=f16 clamp=sym`).
//   y[t, n] = sum_g s[n, g] * sum_{k in g} q[n, k] * x[t, k]      (x bf16, y float32)
//
// The drafter runs a block of 16 positions at a time, so the product is a
// skinny GEMM: one workgroup owns 16 output columns x 16 tokens, and its eight
// waves split the K groups (wave w takes g = w, w + 8, ...): more waves per
// CU keep more loads in flight than four (6.1 against 6.5 us at the drafter
// shape; wider workgroups, which read each activation tile fewer times, left
// CUs idle and were slower). Every workgroup reads the whole activation tile,
// so those reads are made cheap: a wave loads its groups' 16 rows x 256 bytes
// in whole-line pieces (four rows a load, issued before the codes), stores
// them to a wave-private LDS tile (piece p of row r at p ^ r: the fragment
// reads below hit 16 distinct positions) and reads its MFMA fragments from
// there. Loading the fragments straight from global memory, 16-byte pieces
// of 32 lines per load, took 6.1 against 5.3 us. Per group a wave
// runs four v_mfma_f32_16x16x32_bf16 on codes decoded to bf16 (exact), from a
// zero accumulator, then folds that group's partial into its float32 result
// with the column's f16 scale (4 FMAs a lane). Within a group, lane quarter q
// takes the 32 contiguous K positions 32 q .. 32 q + 31 (MFMA i reads 8 q' +
// 0..7 of its window from the lane's 8 i .. 8 i + 7): A and B agree on every
// K, and each lane's codes are two 16-byte loads. The eight waves' results
// meet in LDS and are added in wave order.

#include "common.hpp"
#include "launch.hpp"

namespace i8h {

namespace {

constexpr int kLnKS = 8;                  // waves, each a share of the K groups
constexpr int kLnThreads = 64 * kLnKS;
constexpr int kLnTile = 16;       // output columns and tokens per workgroup
constexpr int kLnBatch = 2;       // groups a wave loads before it multiplies

__device__ __forceinline__ bf16x8 ln_decode(uint32_t lo, uint32_t hi) {
  u32x4 p;
  p[0] = pack_bf16x2(sbyte<0>(lo), sbyte<1>(lo));
  p[1] = pack_bf16x2(sbyte<2>(lo), sbyte<3>(lo));
  p[2] = pack_bf16x2(sbyte<0>(hi), sbyte<1>(hi));
  p[3] = pack_bf16x2(sbyte<2>(hi), sbyte<3>(hi));
  return __builtin_bit_cast(bf16x8, p);
}

__global__ void __launch_bounds__(kLnThreads)
k_linear_i8f16(const uint16_t* __restrict__ x, int T, int K, const int8_t* __restrict__ codes,
               const uint16_t* __restrict__ scales, int N, float* __restrict__ y) {
  __shared__ f32x4 part[kLnKS][kWave];
  // each wave's activation tiles, one per batch slot: 16 rows x 16 pieces of 16 bytes
  __shared__ u32x4 xs[kLnKS][kLnBatch][kLnTile][16];
  const int n0 = blockIdx.x * kLnTile, t0 = blockIdx.y * kLnTile;
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int c = lane % 16, kq = lane / 16;    // column (B) and token (A) of the lane; K quarter
  const int G = K / kGroup;
  const int8_t* crow = codes + (size_t)(n0 + c) * K + 32 * kq;
  const uint16_t* srow = scales + (size_t)(n0 + c) * G;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int g0 = wave; g0 < G; g0 += kLnKS * kLnBatch) {
    // every load of up to kLnBatch groups is issued before the first product:
    // the activation rows (whole lines, into the wave's LDS tile) and the
    // scales, then the codes (the HBM stream)
    u32x4 cv[kLnBatch][2];
    bf16x8 xa[kLnBatch][4];
    float sc[kLnBatch];
#pragma unroll
    for (int b = 0; b < kLnBatch; ++b) {
      const int g = g0 + kLnKS * b;
      if (g < G) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * j + lane / 16, pc = lane % 16;   // rows past T read as zero
          u32x4 v = {0u, 0u, 0u, 0u};
          if (t0 + r < T) v = *reinterpret_cast<const u32x4*>(x + (size_t)(t0 + r) * K + (size_t)g * kGroup + 8 * pc);
          xs[wave][b][r][pc ^ r] = v;
        }
        sc[b] = (float)__builtin_bit_cast(_Float16, srow[g]);
      }
    }
#pragma unroll
    for (int b = 0; b < kLnBatch; ++b) {
      const int g = g0 + kLnKS * b;
      if (g < G) {
        cv[b][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow + (size_t)g * kGroup));
        cv[b][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow + (size_t)g * kGroup + 16));
      }
    }
    // the tile is the wave's own: the wave's stores are ordered before its reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int b = 0; b < kLnBatch; ++b) {
      const int g = g0 + kLnKS * b;
      if (g < G) {
        // MFMA i takes piece 4 kq + i of row (token) c
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[b][i] = __builtin_bit_cast(bf16x8, xs[wave][b][c][(4 * kq + i) ^ c]);
      }
    }
#pragma unroll
    for (int b = 0; b < kLnBatch; ++b) {
      const int g = g0 + kLnKS * b;
      if (g < G) {
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[b][0], ln_decode(cv[b][0][0], cv[b][0][1]), p, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[b][1], ln_decode(cv[b][0][2], cv[b][0][3]), p, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[b][2], ln_decode(cv[b][1][0], cv[b][1][1]), p, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[b][3], ln_decode(cv[b][1][2], cv[b][1][3]), p, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc[b], p[i], acc[i]);
      }
    }
    // the next iteration overwrites the tile: every lane's reads come first
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 r = part[0][lane];
#pragma unroll
    for (int w = 1; w < kLnKS; ++w) {
      const f32x4 o = part[w][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] += o[i];
    }
    // output of the 16x16 tile: lane holds column c, tokens 4 kq .. 4 kq + 3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * kq + i;
      if (t < T) y[(size_t)t * N + n0 + c] = r[i];
    }
  }
}

}  // namespace

hipError_t launch_linear_i8f16(const uint16_t* x, int T, int K, const int8_t* codes, const uint16_t* scales, int N,
                               float* y, hipStream_t st) {
  const dim3 grid(N / kLnTile, cdiv(T, kLnTile));
  k_linear_i8f16<<<grid, kLnThreads, 0, st>>>(x, T, K, codes, scales, N, y);
  return hipGetLastError();
}

}  // namespace i8h
