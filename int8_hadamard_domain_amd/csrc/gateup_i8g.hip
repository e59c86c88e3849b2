// Grouped gate_up in the W8A8 int8 g128 form ("Gemma 4 12B-it · int8 · for
// radiance", header table row "Format"; the int5 card's row "Format" uses
// such activations above 64 rows, so this is the prefill-shaped form):
// int8 codes with one bf16 scale per row and 128 of K (no rotation), int8
// activations with one float32 scale per token and 128 of K.
//   sx[t, g] = amax_g / 127 (IEEE single division), qx = rne(x / sx) clamped to +-127
//   gu[r, n] = sum_g sw[e, n, g] * sx[t, g] * sum_{kk in g} qw[e, n, kk] * qx[t, kk]
//   act[r, i] = gelu_tanh(gu[r, i]) * gu[r, I + i]
// (act stored as float32, or with AT = uint16_t as bf16 rounded to nearest
// even from the float32 value)
//
// Both operands stay int8 all the way into v_mfma_i32_32x32x32_i8: the group
// sums are exact int32 (|sum| <= 128 * 127 * 127 < 2^21), and each is folded
// into the float32 result with sw * sx (convert, multiply, fused add).
//
// At prefill the int8 kernels are bound by the bytes copied global -> LDS,
// so the unit is as large as the registers allow: expert e x (128 gate + the
// matching 128 up columns) x passes of 192 pairs. Per expert the codes then
// stream once (a prefill batch of 2048 tokens x top-8 over 128 experts gives
// 105..154 pairs an expert) and the int8 activation rows are copied once per
// 128 gate columns. Eight waves: wave w takes gate columns 32 (w % 4) .. +31
// and the matching up columns, for the 32-row m-tiles 64 a + 32 (w / 4),
// a = 0..2 (the two waves of a SIMD interleave their m-tiles, so both have
// work however many pairs the pass holds). A wave works one m-tile at a
// time: 8 MFMAs into two int32 tiles, then their fold; its float32 results
// take 96 registers.
//
// Pipeline: K goes in stages of one 128-K group (A 24 KB, B 32 KB, side data
// 1.75 KB) through a 2-slot LDS ring by gfx950's global -> LDS DMA: the copies
// of stage h + 1 run while stage h is multiplied. Rows are 128 bytes, 16-byte
// piece p of row r at position p ^ ((r >> 1) & 7), so the fragment reads of
// 16 consecutive rows hit distinct banks. MFMA k-step s (32 K) takes piece
// 2 s + (lane / 32) of the lane's row for both operands, so A and B agree on
// every k whatever the instruction's lane order within the step.
// The 32x32 result sits in lane l as column l % 32, rows
// 8 (j / 4) + 4 (l / 32) + j % 4.

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

namespace i8h {

namespace {

constexpr int kIThreads = 512;   // 8 waves
constexpr int kICols = 128;      // gate columns per unit (plus as many up)
constexpr int kIRows = 192;      // pass rows
constexpr int kIMt = kIRows / 64; // m-tiles per wave
constexpr int kIXcds = 8;
constexpr int kIRowB = 128;      // bytes per row of a stage (one 128-K group of int8)

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

// the ring: one array per slot, so a copy in flight to one slot does not
// alias reads of the other
__shared__ __attribute__((aligned(16))) uint8_t gA0[kIRows * kIRowB];
__shared__ __attribute__((aligned(16))) uint8_t gA1[kIRows * kIRowB];
__shared__ __attribute__((aligned(16))) uint8_t gB0[2 * kICols * kIRowB];
__shared__ __attribute__((aligned(16))) uint8_t gB1[2 * kICols * kIRowB];
// side data of the slot's group: [0, 256) the dword holding the bf16 scale
// of each code row, [256, 448) the float32 sx of each pass row
__shared__ __attribute__((aligned(16))) uint32_t gC0[2 * kICols + kIRows];
__shared__ __attribute__((aligned(16))) uint32_t gC1[2 * kICols + kIRows];

__device__ __forceinline__ uint32_t g_lds(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)p);
}
// a pointer the caller knows to be wave-uniform, moved to scalar registers
__device__ __forceinline__ const void* g_uniform(const void* p) {
  const uint64_t b = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// one 16- or 4-byte copy per lane, global (uniform base + 32-bit lane offset)
// -> LDS (M0 = the wave's LDS base; lane l's bytes land at base + size * l);
// the kernel waits with vmcnt
// M0 is a register the compiler reserves: it never allocates it, but sets it
// right before its own instructions that read it. Naming it clobbered orders
// these statements against such uses; the compiler still warns that it does
// not preserve reserved registers, which is what is wanted here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void g_dma16(uint32_t off, const void* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void g_dma4(uint32_t off, const void* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
// the same with a 64-bit per-lane address
__device__ __forceinline__ void g_dma4v(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
// s_waitcnt vmcnt(0) with expcnt and lgkmcnt unconstrained (gfx9 field layout)
constexpr int kVmcnt0 = (0x7 << 4) | (0xF << 8);

__device__ __forceinline__ int g_pos(int row, int piece) { return piece ^ ((row >> 1) & 7); }

template <typename AT>
__global__ void __launch_bounds__(kIThreads)
k_gateup_i8g(const int8_t* __restrict__ qx, const float* __restrict__ sx, int K, const int8_t* __restrict__ codes,
             const uint16_t* __restrict__ scales, int E, int N, int k, const int32_t* __restrict__ expert_off,
             const int32_t* __restrict__ sorted_pairs, float* __restrict__ gu, AT* __restrict__ act, int ntiles) {
  // the units of expert e run on XCD e % 8, consecutive in dispatch order
  const int blk = blockIdx.x;
  const int slot = blk / kIXcds;
  const int e = (blk % kIXcds) + kIXcds * (slot / ntiles);
  const int nt = slot % ntiles;
  if (e >= E) return;
  const int r0 = expert_off[e];
  const int m_e = expert_off[e + 1] - r0;
  if (m_e <= 0) return;

  const int I = N / 2, G = K / kGroup;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane % 32, half = lane / 32;
  const int ns = wave % 4, mh = 32 * (wave / 4);
  const int i0 = nt * kICols + 32 * ns;
  const bool live = i0 < I;                       // I % 32 == 0: a live wave has all 32 columns
  const int rg = 32 * ns + col, ru = kICols + 32 * ns + col;   // this lane's code rows in a B stage
  const uint32_t la[2] = {g_lds(gA0), g_lds(gA1)};
  const uint32_t lb[2] = {g_lds(gB0), g_lds(gB1)};
  const uint32_t lc[2] = {g_lds(gC0), g_lds(gC1)};

  // code rows this lane copies: instruction q fills B rows 8 (4 wave + q) ..
  // +7, lane l row + l / 8 at position l % 8 (rows past I repeat the
  // expert's row 0); offsets from the expert's first code byte
  const void* cbase_e = g_uniform(codes + (size_t)e * N * K);
  uint32_t boff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 8 * (4 * wave + q) + lane / 8;
    const int gi = nt * kICols + (row % kICols);
    const int n = gi < I ? (row < kICols ? gi : I + gi) : 0;
    boff[q] = (uint32_t)(n * K + 16 * g_pos(row, lane % 8));
  }
  // waves 0..3: the scale dword of code row 64 wave + lane (element index
  // srow + g; the bf16 is its half (srow + g) & 1)
  int64_t srow = 0;
  if (wave < 4) {
    const int row = 64 * wave + lane;
    const int gi = nt * kICols + (row % kICols);
    const int n = gi < I ? (row < kICols ? gi : I + gi) : 0;
    srow = ((int64_t)e * N + n) * G;
  }
  const int par_g = (int)((((int64_t)e * N + (live ? i0 + col : 0)) * G) & 1);
  const int par_u = (int)((((int64_t)e * N + (live ? I + i0 + col : 0)) * G) & 1);
  const void* qx_u = g_uniform(qx);
  const void* sx_u = g_uniform(sx);

  for (int mb = 0; mb < m_e; mb += kIRows) {
    const int rows = min(kIRows, m_e - mb);
    // activation rows this lane copies: instruction q fills pass rows
    // 8 (3 wave + q) + lane / 8 (rows past the pass repeat its last row);
    // only blocks holding pass rows are copied
    uint32_t aoff[kIMt];
    int nca = 0;
#pragma unroll
    for (int q = 0; q < kIMt; ++q) {
      const int row = 8 * (kIMt * wave + q) + lane / 8;
      const int t = sorted_pairs[r0 + mb + min(row, rows - 1)] / k;
      aoff[q] = (uint32_t)(t * K + 16 * g_pos(row, lane % 8));
      if (8 * (kIMt * wave + q) < rows) ++nca;
    }
    nca = __builtin_amdgcn_readfirstlane(nca);
    // waves 4..6: sx of pass row 64 (wave - 4) + lane
    uint32_t xoff = 0;
    if (wave >= 4 && wave < 4 + kIRows / 64) {
      const int row = 64 * (wave - 4) + lane;
      const int t = sorted_pairs[r0 + mb + min(row, rows - 1)] / k;
      xoff = (uint32_t)(t * G) * 4u;
    }

    // group g into ring slot sl
    auto issue = [&](int g, int sl) __attribute__((always_inline)) {
      const uint32_t kb = (uint32_t)(g * kIRowB);
#pragma unroll
      for (int q = 0; q < kIMt; ++q)
        if (q < nca) g_dma16(aoff[q] + kb, qx_u, la[sl] + (kIMt * wave + q) * (8 * kIRowB));
#pragma unroll
      for (int q = 0; q < 4; ++q) g_dma16(boff[q] + kb, cbase_e, lb[sl] + (4 * wave + q) * (8 * kIRowB));
      if (wave < 4)
        g_dma4v(scales + ((srow + g) & ~(int64_t)1), lc[sl] + 64 * 4 * wave);
      else if (wave < 4 + kIRows / 64)
        g_dma4(xoff + 4u * (uint32_t)g, sx_u, lc[sl] + 4 * (2 * kICols + 64 * (wave - 4)));
    };

    f32x16 acc[kIMt][2];
#pragma unroll
    for (int a = 0; a < kIMt; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[a][c][j] = 0.0f;

    auto stage = [&](int g, const uint8_t* abuf, const uint8_t* bbuf, const uint32_t* cbuf, int next_slot)
        __attribute__((always_inline)) {
      if (g >= G) return;
      __builtin_amdgcn_s_waitcnt(kVmcnt0);             // this wave's copies of group g
      __builtin_amdgcn_s_barrier();                    // ... and every other wave's; slot g - 1 is free
      if (g + 1 < G) issue(g + 1, next_slot);
      if (!live) return;
      i32x4 bgf[4], buf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bgf[s] = *reinterpret_cast<const i32x4*>(&bbuf[rg * kIRowB + 16 * g_pos(rg, 2 * s + half)]);
        buf[s] = *reinterpret_cast<const i32x4*>(&bbuf[ru * kIRowB + 16 * g_pos(ru, 2 * s + half)]);
      }
      auto half_bf16 = [](uint32_t w, int odd) { return __uint_as_float(odd ? (w & 0xffff0000u) : (w << 16)); };
      const float wg = half_bf16(cbuf[rg], (par_g + g) & 1);
      const float wu = half_bf16(cbuf[ru], (par_u + g) & 1);
#pragma unroll
      for (int a = 0; a < kIMt; ++a) {
        const int m0 = 64 * a + mh;
        if (m0 >= rows) break;
        const int m = m0 + col;
        i32x16 tg = {}, tu = {};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const i32x4 av = *reinterpret_cast<const i32x4*>(&abuf[m * kIRowB + 16 * g_pos(m, 2 * s + half)]);
          tg = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bgf[s], tg, 0, 0, 0);
          tu = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, buf[s], tu, 0, 0, 0);
        }
        // sx of the result rows m0 + 8 q + 4 half + i
        const float* fx = reinterpret_cast<const float*>(cbuf + 2 * kICols);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 f = *reinterpret_cast<const f32x4*>(&fx[m0 + 8 * q + 4 * half]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[a][0][4 * q + i] = fmaf((float)tg[4 * q + i], wg * f[i], acc[a][0][4 * q + i]);
            acc[a][1][4 * q + i] = fmaf((float)tu[4 * q + i], wu * f[i], acc[a][1][4 * q + i]);
          }
        }
        // one m-tile's two int32 tiles live at a time: the fold is pinned
        // here, before the next m-tile's products (the compiler would
        // otherwise sink it past them and hold every m-tile's int32 tiles)
        asm volatile("" : "+v"(acc[a][0]), "+v"(acc[a][1]));
      }
    };

    __builtin_amdgcn_s_barrier();  // nobody still reads the ring of the previous pass
    issue(0, 0);
    for (int g = 0; g < G; g += 2) {   // group g uses slot g % 2, fixed at compile time
      stage(g, gA0, gB0, gC0, 1);
      stage(g + 1, gA1, gB1, gC1, 0);
    }
    if (live) {
      // uniform bases and 32-bit lane offsets, opaque so the compiler does
      // not hoist the store addresses of every pass out of the pass loop
      AT* act_b = act ? act + (size_t)(r0 + mb) * I : nullptr;
      float* gu_b = gu ? gu + (size_t)(r0 + mb) * N : nullptr;
#pragma unroll
      for (int a = 0; a < kIMt; ++a) {
        const int m0 = 64 * a + mh;
        if (m0 >= rows) break;
        uint32_t go = (uint32_t)((m0 + 4 * half) * N + i0 + col), ao = (uint32_t)((m0 + 4 * half) * I + i0 + col);
        asm volatile("" : "+v"(go), "+v"(ao));
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int dm = 8 * (j / 4) + (j % 4);
          if (m0 + 4 * half + dm < rows) {
            const float gv = acc[a][0][j], uv = acc[a][1][j];
            if (gu_b) {
              gu_b[go + (uint32_t)(dm * N)] = gv;
              gu_b[go + (uint32_t)(dm * N + I)] = uv;
            }
            if (act_b) put_act(act_b, ao + (uint32_t)(dm * I), gelu_tanh(gv) * uv);
          }
        }
      }
    }
  }
}

// Activation quantizer: 16 lanes per (token, group), 8 values a lane.
constexpr int kQThreads = 256;

__global__ void __launch_bounds__(kQThreads)
k_i8_act_quant(const uint16_t* __restrict__ x, int T, int K, int8_t* __restrict__ qx, float* __restrict__ sx) {
  const int G = K / kGroup;
  const int64_t grp = (int64_t)blockIdx.x * (kQThreads / 16) + threadIdx.x / 16;
  const int j = threadIdx.x % 16;
  const bool valid = grp < (int64_t)T * G;
  const int64_t t = valid ? grp / G : 0;
  const int g = valid ? (int)(grp % G) : 0;
  u32x4 w = {0u, 0u, 0u, 0u};
  if (valid) w = *reinterpret_cast<const u32x4*>(x + t * K + g * kGroup + 8 * j);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, xor_lane<1>(amax));
  amax = fmaxf(amax, xor_lane<2>(amax));
  amax = fmaxf(amax, xor_lane<4>(amax));
  amax = fmaxf(amax, xor_lane<8>(amax));
  const float s = amax / 127.0f;                 // IEEE single division
  uint32_t out[2] = {0u, 0u};
  if (s != 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = fminf(fmaxf(__builtin_rintf(v[i] / s), -127.0f), 127.0f);   // nearest even
      out[i / 4] |= ((uint32_t)(int)q & 0xffu) << (8 * (i % 4));
    }
  }
  if (valid) {
    *reinterpret_cast<u32x2*>(qx + t * K + g * kGroup + 8 * j) = u32x2{out[0], out[1]};
    if (j == 0) sx[t * G + g] = s;
  }
}

}  // namespace

hipError_t launch_i8_act_quant(const uint16_t* x, int T, int K, int8_t* qx, float* sx, hipStream_t st) {
  const int64_t groups = (int64_t)T * (K / kGroup);
  const int per = kQThreads / 16;
  const int grid = (int)((groups + per - 1) / per);
  k_i8_act_quant<<<grid, kQThreads, 0, st>>>(x, T, K, qx, sx);
  return hipGetLastError();
}

hipError_t launch_gateup_i8g(const int8_t* qx, const float* sx, int T, int K, const int8_t* codes,
                             const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                             const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16, hipStream_t st) {
  (void)T;
  const int ntiles = cdiv(N / 2, kICols);
  const int grid = cdiv(E, kIXcds) * kIXcds * ntiles;
  if (act_bf16)
    k_gateup_i8g<<<grid, kIThreads, 0, st>>>(qx, sx, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu,
                                             static_cast<uint16_t*>(act), ntiles);
  else
    k_gateup_i8g<<<grid, kIThreads, 0, st>>>(qx, sx, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu,
                                             static_cast<float*>(act), ntiles);
  return hipGetLastError();
}

}  // namespace i8h
