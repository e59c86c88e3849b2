// Grouped gate_up for few pairs per expert (a verify batch: 128 tokens x
// top-8 over 128 experts is about 8 pairs an expert), for both weight formats.
//
// int8 Hadamard-domain (int8 card, model table row "Weights"): int8 codes
// -127..127, one bf16 scale per row and 128 of K, activations rotated bf16.
//   gu[r, n] = sum_g s[e, n, g] * sum_{kk in g} q[e, n, kk] * x_rot[t, kk]
// FP8 E4M3 128x128 blocks (FP8 card, model table row "Weights"): one bf16
// scale per block, activations quantized per token and 128 of K (float32
// factor sx, E4M3 codes handed over as their exact bf16 values).
//   gu[r, n] = sum_g (sw[e, n/128, g] * sx[t, g]) * sum_{kk in g} qw * qx
// Both: act[r, i] = gelu_tanh(gu[r, i]) * gu[r, I + i], stored as float32 or
// (AT = uint16_t) as bf16 rounded to nearest even from the float32 value.
//
// With a handful of pairs per expert the step is a stream of the touched
// experts' codes, and what bounds it is how many bytes each CU keeps in
// flight and how long a unit waits to fill its pipeline. So the unit is small
// and three workgroups share a CU (one fills or drains while the others
// stream): unit = expert e x (64 gate + the matching 64 up columns) x passes
// of 64 pairs; 4 waves, wave w takes gate columns 32 (w & 1) .. +31 and the
// matching up columns for the m-tile w >> 1 (32 pass rows). An expert with at
// most 32 pairs (most of them, at a verify batch) has one m-tile, and then the
// waves w >> 1 = 1 take k-steps 2 and 3 of every stage instead, for the same
// columns and rows as the waves w >> 1 = 0 (k-steps 0 and 1): every wave
// decodes half of its columns' codes, instead of two waves decoding all of
// them while two idle, and the two partial sums of an output are added in a
// fixed order at the end (the workgroup picks the form once, from its
// expert's pair count, so each form is compiled on its own). K goes in stages
// of 64 through a 3-slot LDS ring (A 8 KB, B 8 KB, side data 512 B a slot:
// 49.5 KB a workgroup, so three share a CU) by gfx950's global -> LDS DMA,
// two stages ahead. Each 128-K group's products accumulate from zero and are
// folded into the float32 result with the group's scale (int8: the column's;
// E4M3: block scale times the pass row's sx); v_mfma_f32_32x32x16_bf16 on
// codes decoded to bf16 exactly (int8 by byte converts, E4M3 two codes an
// instruction by v_cvt_scalef32_pk_bf16_fp8 with scale 1: both fit bf16's
// significand).
//
// Stage layouts as in the larger kernels: A piece p (8 bf16) of row r (128
// bytes) at p ^ ((r >> 1) & 7), B piece p (16 codes) of row r (64 bytes) at
// p ^ ((r >> 2) & 3). Within a 64-K stage, MFMA k-step s takes
// k = 32 half + 8 s .. +7 in the lanes of half `half` (lane / 32): a B lane
// reads one contiguous 32-byte span of its row (pieces 2 half, 2 half + 1;
// sixteen consecutive rows then cover all 64 banks) and an A lane piece
// 4 half + s, so both operands agree on every k.

#include "common.hpp"
#include "launch.hpp"

namespace i8h {

namespace {

constexpr int kSThreads = 256;   // 4 waves
constexpr int kSGate = 64;       // gate columns per unit (plus as many up)
constexpr int kSRows = 64;       // pass rows
constexpr int kSStageK = 64;
constexpr int kSXcds = 8;

typedef __attribute__((address_space(3))) void lds_void_t;

// one array per slot: a copy in flight to one slot does not alias reads of another
__shared__ __attribute__((aligned(16))) uint16_t sA0[kSRows * kSStageK];
__shared__ __attribute__((aligned(16))) uint16_t sA1[kSRows * kSStageK];
__shared__ __attribute__((aligned(16))) uint16_t sA2[kSRows * kSStageK];
__shared__ __attribute__((aligned(16))) uint8_t sB0[2 * kSGate * kSStageK];
__shared__ __attribute__((aligned(16))) uint8_t sB1[2 * kSGate * kSStageK];
__shared__ __attribute__((aligned(16))) uint8_t sB2[2 * kSGate * kSStageK];
// side data of the group whose second stage this slot holds (second stages
// land in any slot): int8 -> the dword holding the bf16 scale of each of the
// unit's 128 code rows; E4M3 -> the sx of the 64 pass rows, then 64 dwords
// holding the gate (even lanes) and up (odd lanes) block scales
__shared__ __attribute__((aligned(16))) uint32_t sC0[2 * kSGate];
__shared__ __attribute__((aligned(16))) uint32_t sC1[2 * kSGate];
__shared__ __attribute__((aligned(16))) uint32_t sC2[2 * kSGate];

constexpr int s_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

__device__ __forceinline__ uint32_t s_lds(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)p);
}
// one 16- or 4-byte copy per lane, global -> LDS (M0 = the wave's LDS base;
// lane l's bytes land at base + size * l); the kernel waits with vmcnt
// M0 is a register the compiler reserves: it never allocates it, but sets it
// right before its own instructions that read it. Naming it clobbered orders
// these statements against such uses; the compiler still warns that it does
// not preserve reserved registers, which is what is wanted here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void s_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void s_dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
// s_waitcnt vmcnt(n) for a wave-uniform count known at run time (0..10)
__device__ __forceinline__ void s_wait_dyn(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(s_vm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(s_vm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(s_vm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(s_vm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(s_vm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(s_vm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(s_vm(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(s_vm(7)); break;
    case 8: __builtin_amdgcn_s_waitcnt(s_vm(8)); break;
    case 9: __builtin_amdgcn_s_waitcnt(s_vm(9)); break;
    default: __builtin_amdgcn_s_waitcnt(s_vm(10)); break;
  }
}

__device__ __forceinline__ int sa_pos(int row, int piece) { return piece ^ ((row >> 1) & 7); }
__device__ __forceinline__ int sb_pos(int row, int piece) { return piece ^ ((row >> 2) & 3); }

enum class SFmt { I8, E4M3 };

template <SFmt F>
__device__ __forceinline__ bf16x8 s_decode(uint32_t lo, uint32_t hi) {
  u32x4 p;
  if constexpr (F == SFmt::I8) {
    p[0] = pack_bf16x2(sbyte<0>(lo), sbyte<1>(lo));
    p[1] = pack_bf16x2(sbyte<2>(lo), sbyte<3>(lo));
    p[2] = pack_bf16x2(sbyte<0>(hi), sbyte<1>(hi));
    p[3] = pack_bf16x2(sbyte<2>(hi), sbyte<3>(hi));
  } else {
    // E4M3 -> bf16 is exact; the scaled pair conversion with scale 1 turns
    // two codes into two bf16 values in one instruction
    p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
    p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
    p[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
    p[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  }
  return __builtin_bit_cast(bf16x8, p);
}

template <SFmt F, bool KS, typename AT>
__device__ __forceinline__ void skinny_body(const uint16_t* __restrict__ xa, const float* __restrict__ sx, int K,
                                            const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                            int E, int N, int k, const int32_t* __restrict__ expert_off,
                                            const int32_t* __restrict__ sorted_pairs, float* __restrict__ gu,
                                            AT* __restrict__ act, int ntiles) {
  // the units of expert e run on XCD e % 8, consecutive in dispatch order
  const int blk = blockIdx.x;
  const int slot = blk / kSXcds;
  const int e = (blk % kSXcds) + kSXcds * (slot / ntiles);
  const int nt = slot % ntiles;
  if (e >= E) return;
  const int r0 = expert_off[e];
  const int m_e = expert_off[e + 1] - r0;
  if (m_e <= 0) return;

  const int I = N / 2, G = K / kGroup, NB = N / kGroup;
  const int S = 2 * G;                            // stages per pass
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane % 32, half = lane / 32;
  const int ns = wave & 1, mw = 32 * (wave >> 1);
  const int i0 = nt * kSGate + 32 * ns;
  const bool live = i0 < I;                       // I % 32 == 0: a live wave has all 32 columns
  const int rg = 32 * ns + col, ru = kSGate + 32 * ns + col;   // this lane's code rows in a B stage
  const uint32_t la[3] = {s_lds(sA0), s_lds(sA1), s_lds(sA2)};
  const uint32_t lb[3] = {s_lds(sB0), s_lds(sB1), s_lds(sB2)};
  const uint32_t lc[3] = {s_lds(sC0), s_lds(sC1), s_lds(sC2)};

  // code rows this lane copies: instruction q fills B rows 16 (2 wave + q) .. +15,
  // lane l row + l / 4 at position l % 4 (rows past I repeat the expert's row 0)
  size_t bsrc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 16 * (2 * wave + q) + lane / 4;
    const int gi = nt * kSGate + (row % kSGate);
    const int n = gi < I ? (row < kSGate ? gi : I + gi) : 0;
    bsrc[q] = ((size_t)e * N + n) * K + 16 * sb_pos(row, lane % 4);
  }
  // side data copied with the second stage of group g (dword of element
  // index cbase + g; the wanted bf16 is its half (cbase + g) & 1):
  //   int8, waves 0, 1: the scale of code row 64 wave + lane
  //   E4M3, wave 0: sx of pass row lane (set per pass); wave 1: the gate
  //   (even lanes) or up (odd lanes) block scale of the unit's 64 columns,
  //   which lie in one 128-column block each
  int64_t cbase = 0;
  if constexpr (F == SFmt::I8) {
    const int row = 64 * (wave & 1) + lane;
    const int gi = nt * kSGate + (row % kSGate);
    const int n = gi < I ? (row < kSGate ? gi : I + gi) : 0;
    cbase = ((int64_t)e * N + n) * G;
  } else {
    const int gi = nt * kSGate;                   // < I for every launched tile
    const int nb = (lane & 1) ? (I + gi) / kGroup : gi / kGroup;
    cbase = ((int64_t)e * NB + nb) * G;
  }
  int par_g, par_u;
  if constexpr (F == SFmt::I8) {
    par_g = (int)((((int64_t)e * N + (live ? i0 + col : 0)) * G) & 1);
    par_u = (int)((((int64_t)e * N + (live ? I + i0 + col : 0)) * G) & 1);
  } else {
    par_g = (int)((((int64_t)e * NB + (nt * kSGate) / kGroup) * G) & 1);
    par_u = (int)((((int64_t)e * NB + (I + nt * kSGate) / kGroup) * G) & 1);
  }

  for (int mb = 0; mb < m_e; mb += kSRows) {
    const int rows = min(kSRows, m_e - mb);
    // KS: the expert has at most 32 pairs, so this is its only pass and it
    // has one m-tile; the waves w >> 1 = 1 then take k-steps 2 and 3 of every
    // stage for the same columns and rows, and their partial sums join the
    // first waves' at the end
    constexpr bool ksplit = KS;
    const int mt = ksplit ? 0 : mw;               // first pass row of the wave's m-tile
    const int kh = wave >> 1;                     // with ksplit: k-steps 2 kh and 2 kh + 1
    const bool busy = live && rows > mt;          // the wave has live rows in this pass
    // activation rows this lane copies: instruction q fills pass rows
    // 8 (2 wave + q) .. +7, lane l row + l / 8 at position l % 8; only blocks
    // holding pass rows are copied (rows past the pass repeat its last row)
    int asrc[2];
    int nca = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = 8 * (2 * wave + q) + lane / 8;
      const int t = sorted_pairs[r0 + mb + min(row, rows - 1)] / k;
      asrc[q] = t * K + 8 * sa_pos(row, lane % 8);
      if (8 * (2 * wave + q) < rows) ++nca;
    }
    nca = __builtin_amdgcn_readfirstlane(nca);
    int xtok = 0;                                 // E4M3, wave 0: token of pass row lane
    if constexpr (F == SFmt::E4M3) xtok = sorted_pairs[r0 + mb + min(lane, rows - 1)] / k;
    // copies of stage h by this wave
    auto dmas = [&](int h) { return nca + 2 + ((wave < 2 && (h & 1)) ? 1 : 0); };
    // stage h into ring slot sl (== h % 3, given as a constant by the caller)
    auto issue = [&](int h, int sl) __attribute__((always_inline)) {
      const int koff = h * kSStageK;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (q < nca) s_dma16(xa + asrc[q] + koff, la[sl] + (2 * wave + q) * (8 * kSStageK * 2));
#pragma unroll
      for (int q = 0; q < 2; ++q) s_dma16(codes + bsrc[q] + koff, lb[sl] + (2 * wave + q) * (16 * kSStageK));
      if ((h & 1) && wave < 2) {
        if (F == SFmt::E4M3 && wave == 0)
          s_dma4(sx + (size_t)xtok * G + h / 2, lc[sl]);
        else
          s_dma4(scales + ((cbase + h / 2) & ~(int64_t)1), lc[sl] + 64 * 4 * wave);
      }
    };

    f32x16 acc[2], tmp[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[c][j] = 0.0f;

    auto stage = [&](int h, const uint16_t* abuf, const uint8_t* bbuf, const uint32_t* cbuf, int next_slot)
        __attribute__((always_inline)) {
      if (h >= S) return;
      // this wave's copies of stage h are in LDS (those of the stage issued
      // after it may stay in flight), then every other wave's
      s_wait_dyn(h + 1 < S ? dmas(h + 1) : 0);
      __builtin_amdgcn_s_barrier();
      if (h + 2 < S) issue(h + 2, next_slot);     // the slot of stage h - 1, now free
      if (!busy) return;
      if ((h & 1) == 0) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int j = 0; j < 16; ++j) tmp[c][j] = 0.0f;
      }
      // the lane's 32 codes of the stage (k = 32 half .. +31): pieces 2 half
      // and 2 half + 1 of its gate and up rows
      const int m = mt + col;
      if constexpr (KS) {
        // k-steps 2 kh, 2 kh + 1: piece 2 half + kh of the lane's code rows
        const u32x4 g4 = *reinterpret_cast<const u32x4*>(&bbuf[rg * kSStageK + 16 * sb_pos(rg, 2 * half + kh)]);
        const u32x4 u4 = *reinterpret_cast<const u32x4*>(&bbuf[ru * kSStageK + 16 * sb_pos(ru, 2 * half + kh)]);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int s = 2 * kh + s2;
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(&abuf[m * kSStageK + 8 * sa_pos(m, 4 * half + s)]);
          tmp[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, s_decode<F>(g4[2 * s2], g4[2 * s2 + 1]), tmp[0], 0,
                                                           0, 0);
          tmp[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, s_decode<F>(u4[2 * s2], u4[2 * s2 + 1]), tmp[1], 0,
                                                           0, 0);
        }
      } else {
        u32x4 cg[2], cu[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          cg[q] = *reinterpret_cast<const u32x4*>(&bbuf[rg * kSStageK + 16 * sb_pos(rg, 2 * half + q)]);
          cu[q] = *reinterpret_cast<const u32x4*>(&bbuf[ru * kSStageK + 16 * sb_pos(ru, 2 * half + q)]);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(&abuf[m * kSStageK + 8 * sa_pos(m, 4 * half + s)]);
          const u32x4& g4 = cg[s / 2];
          const u32x4& u4 = cu[s / 2];
          tmp[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, s_decode<F>(g4[2 * (s % 2)], g4[2 * (s % 2) + 1]),
                                                           tmp[0], 0, 0, 0);
          tmp[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, s_decode<F>(u4[2 * (s % 2)], u4[2 * (s % 2) + 1]),
                                                           tmp[1], 0, 0, 0);
        }
      }
      if (h & 1) {
        const int g = h / 2;
        auto half_bf16 = [](uint32_t w, int odd) { return __uint_as_float(odd ? (w & 0xffff0000u) : (w << 16)); };
        if constexpr (F == SFmt::I8) {
          const float sg = half_bf16(cbuf[rg], (par_g + g) & 1), su = half_bf16(cbuf[ru], (par_u + g) & 1);
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            acc[0][j] = fmaf(tmp[0][j], sg, acc[0][j]);
            acc[1][j] = fmaf(tmp[1][j], su, acc[1][j]);
          }
        } else {
          const float wg = half_bf16(cbuf[kSRows], (par_g + g) & 1);
          const float wu = half_bf16(cbuf[kSRows + 1], (par_u + g) & 1);
          // sx of the lane's result rows mt + 4 half + 8 (j / 4) + j % 4
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 f = *reinterpret_cast<const f32x4*>(&cbuf[mt + 4 * half + 8 * q]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc[0][4 * q + i] = fmaf(tmp[0][4 * q + i], wg * f[i], acc[0][4 * q + i]);
              acc[1][4 * q + i] = fmaf(tmp[1][4 * q + i], wu * f[i], acc[1][4 * q + i]);
            }
          }
        }
      }
    };

    __builtin_amdgcn_s_barrier();  // nobody still reads the ring of the previous pass
    issue(0, 0);
    if (S > 1) issue(1, 1);
    for (int hb = 0; hb < S; hb += 3) {      // stage h uses slot h % 3, fixed at compile time
      stage(hb + 0, sA0, sB0, sC0, 2);
      stage(hb + 1, sA1, sB1, sC1, 0);
      stage(hb + 2, sA2, sB2, sC2, 1);
    }
    if constexpr (KS) {
      // the second waves' partial sums join the first waves' (same columns,
      // same rows) through the A slots of the ring, free once every wave is
      // past its last stage; the next pass starts with a barrier
      __syncthreads();
      float* xch = reinterpret_cast<float*>(ns ? sA1 : sA0);
      if (kh == 1 && busy) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int j = 0; j < 16; ++j) xch[(16 * c + j) * kWave + lane] = acc[c][j];
      }
      __syncthreads();
      if (kh == 0 && busy) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[c][j] += xch[(16 * c + j) * kWave + lane];
      }
    }
    if (busy && !(ksplit && kh == 1)) {
      // uniform bases and 32-bit lane offsets, opaque so the compiler does
      // not hoist the store addresses of every pass out of the pass loop
      AT* act_b = act ? act + (size_t)(r0 + mb) * I : nullptr;
      float* gu_b = gu ? gu + (size_t)(r0 + mb) * N : nullptr;
      uint32_t go = (uint32_t)((mt + 4 * half) * N + i0 + col), ao = (uint32_t)((mt + 4 * half) * I + i0 + col);
      asm volatile("" : "+v"(go), "+v"(ao));
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int dm = 8 * (j / 4) + (j % 4);
        if (mt + 4 * half + dm < rows) {
          const float gv = acc[0][j], uv = acc[1][j];
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

// the block's expert has 1..32 pairs (one pass with one m-tile): the split form
__device__ __forceinline__ bool skinny_split(int E, const int32_t* __restrict__ expert_off, int ntiles) {
  const int slot = blockIdx.x / kSXcds;
  const int e = (blockIdx.x % kSXcds) + kSXcds * (slot / ntiles);
  if (e >= E) return false;
  const int m_e = expert_off[e + 1] - expert_off[e];
  return m_e <= 32;
}

template <typename AT>
__global__ void __launch_bounds__(kSThreads, 3)
k_gateup_i8h_skinny(const uint16_t* __restrict__ xa, int K, const uint8_t* __restrict__ codes,
                    const uint16_t* __restrict__ scales, int E, int N, int k,
                    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ sorted_pairs,
                    float* __restrict__ gu, AT* __restrict__ act, int ntiles) {
  if (skinny_split(E, expert_off, ntiles))
    skinny_body<SFmt::I8, true>(xa, nullptr, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu, act, ntiles);
  else
    skinny_body<SFmt::I8, false>(xa, nullptr, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu, act, ntiles);
}

template <typename AT>
__global__ void __launch_bounds__(kSThreads, 3)
k_gateup_fp8_skinny(const uint16_t* __restrict__ xq, const float* __restrict__ sx, int K,
                    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int E, int N, int k,
                    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ sorted_pairs,
                    float* __restrict__ gu, AT* __restrict__ act, int ntiles) {
  if (skinny_split(E, expert_off, ntiles))
    skinny_body<SFmt::E4M3, true>(xq, sx, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu, act, ntiles);
  else
    skinny_body<SFmt::E4M3, false>(xq, sx, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu, act, ntiles);
}

}  // namespace

hipError_t launch_gateup_i8h_skinny(const uint16_t* xrot, int T, int K, const int8_t* codes,
                                    const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                    const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16,
                                    hipStream_t st) {
  (void)T;
  const int ntiles = cdiv(N / 2, kSGate);
  const int grid = cdiv(E, kSXcds) * kSXcds * ntiles;
  const uint8_t* q = reinterpret_cast<const uint8_t*>(codes);
  if (act_bf16)
    k_gateup_i8h_skinny<<<grid, kSThreads, 0, st>>>(xrot, K, q, scales, E, N, k, expert_off, sorted_pairs, gu,
                                                    static_cast<uint16_t*>(act), ntiles);
  else
    k_gateup_i8h_skinny<<<grid, kSThreads, 0, st>>>(xrot, K, q, scales, E, N, k, expert_off, sorted_pairs, gu,
                                                    static_cast<float*>(act), ntiles);
  return hipGetLastError();
}

hipError_t launch_gateup_fp8_skinny(const uint16_t* xq, const float* sx, int T, int K, const uint8_t* codes,
                                    const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                    const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16,
                                    hipStream_t st) {
  (void)T;
  const int ntiles = cdiv(N / 2, kSGate);
  const int grid = cdiv(E, kSXcds) * kSXcds * ntiles;
  if (act_bf16)
    k_gateup_fp8_skinny<<<grid, kSThreads, 0, st>>>(xq, sx, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu,
                                                    static_cast<uint16_t*>(act), ntiles);
  else
    k_gateup_fp8_skinny<<<grid, kSThreads, 0, st>>>(xq, sx, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu,
                                                    static_cast<float*>(act), ntiles);
  return hipGetLastError();
}

}  // namespace i8h
