// Verify/prefill-shaped grouped gate_up on bf16 MFMA, for both weight formats.
//
// int8 Hadamard-domain (int8 card, model table row "Weights"): int8 codes in
// -127..127, one bf16 scale per row and 128 of K; activations rotated bf16.
//   gu[r, n] = sum_g s[e, n, g] * sum_{kk in g} q[e, n, kk] * x_rot[t, kk]
// FP8 E4M3 128x128 blocks (FP8 card, model table row "Weights"): one bf16
// scale per block; activations quantized per token and 128 of K (float32
// scale sx, E4M3 codes qx, handed over here as their exact bf16 values).
//   gu[r, n] = sum_g (sw[e, n/128, g] * sx[t, g]) * sum_{kk in g} qw * qx
// Both: act[r, i] = gelu_tanh(gu[r, i]) * gu[r, I + i], stored as float32 or
// (AT = uint16_t) as bf16 rounded to nearest even from the float32 value.
//
// Work unit = (expert e, 128 gate rows + the 128 matching up rows). Blocks
// are mapped so that the units of one expert run on one XCD (the hardware
// hands consecutive workgroups to the 8 XCDs in turn) and share its L2 for
// the expert's activation rows. A unit walks the expert's pairs in passes of
// 128 rows, so each code byte leaves HBM once per pass. Eight waves (two per
// SIMD: one wave's MFMAs overlap the other's converts and folds) split the
// unit: wave w owns gate rows i0..i0+31 and up rows I+i0..I+i0+31 with
// i0 = 32 (w % 4), for pass rows 64 (w / 4) .. +63 (two m-tiles), so the gate
// and up values of an output meet in one lane.
//
// Pipeline: K is cut into stages of 64 (half a scale group). Everything a
// stage needs travels global -> LDS on gfx950's DMA path (global_load_lds: no
// registers held while in flight) into a ring of 4 LDS slots, three stages
// ahead of the one being multiplied: both operands as 16-byte pieces
// XOR-swizzled by row so that fragment reads hit distinct banks, and, with
// the second stage of each group, the group's scales (int8) or block scales
// and per-row activation factors (E4M3) as aligned dwords. The copies are
// issued from inline assembly: the loop then holds no memory operation the
// compiler tracks, and each stage waits for exactly its own copies
// (s_waitcnt vmcnt(8): the copies of the two stages issued after it may stay
// in flight) before a workgroup barrier. v_mfma_f32_32x32x16_bf16
// accumulates a whole 128-K group into a temporary tile that is then folded
// into the float32 result with the group's scale (main += tmp * s); scaling
// the codes first would round each weight to bf16. Codes become bf16
// exactly: int8 by sign-extended byte converts (|q| <= 127 fits bf16's 8
// significand bits), E4M3 two codes an instruction by the scaled pair
// conversion v_cvt_scalef32_pk_bf16_fp8 with scale 1 (3 significand bits).
//
// MFMA operands (32x32x16 bf16): lane l feeds 8 values of row (A) or column
// (B) l % 32 for step s; within a 64-K stage the lanes of half h = l / 32
// take k = 32 h + 8 s + j, so a B lane reads its stage's codes as one
// contiguous 32-byte span (16 consecutive rows then cover all 64 LDS banks)
// and an A lane piece 4 h + s. The 32x32 result sits in lane l as column
// l % 32, rows 8 (j / 4) + 4 (l / 32) + j % 4.

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace i8h {

enum class WFmt { I8, E4M3 };

constexpr int kGThreads = 512;
constexpr int kGateRows = 128;    // gate rows per unit (plus as many up rows)
constexpr int kPassRows = 128;    // pairs per m-pass
constexpr int kMTiles = 2;        // m-tiles of 32 per wave
constexpr int kStageK = 64;       // K per pipeline stage
constexpr int kSlots = 4;         // LDS ring depth (3 stages in flight)
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediates (gfx9 layout: vmcnt [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]); unconstrained fields at their maximum
constexpr int wait_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

template <WFmt F>
__device__ __forceinline__ bf16x8 decode8(uint32_t lo, uint32_t hi) {
  u32x4 p;
  if constexpr (F == WFmt::I8) {
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

// The LDS ring: one array per slot, so the compiler can tell that a DMA in
// flight to one slot does not alias the reads of another (with a single
// indexed array it waits for every copy before any LDS read).
__shared__ __attribute__((aligned(16))) uint16_t gA0[kPassRows * kStageK];
__shared__ __attribute__((aligned(16))) uint16_t gA1[kPassRows * kStageK];
__shared__ __attribute__((aligned(16))) uint16_t gA2[kPassRows * kStageK];
__shared__ __attribute__((aligned(16))) uint16_t gA3[kPassRows * kStageK];
__shared__ __attribute__((aligned(16))) uint8_t gB0[2 * kGateRows * kStageK];
__shared__ __attribute__((aligned(16))) uint8_t gB1[2 * kGateRows * kStageK];
__shared__ __attribute__((aligned(16))) uint8_t gB2[2 * kGateRows * kStageK];
__shared__ __attribute__((aligned(16))) uint8_t gB3[2 * kGateRows * kStageK];
// per-group side data, copied with the second (odd) stage of the group into
// the slot of that stage: int8 -> the dword holding the bf16 scale of each of
// the unit's 256 code rows; E4M3 -> 128 float row factors, then the dwords
// holding the block scales of the 4 column slices (gate, up)
__shared__ __attribute__((aligned(16))) uint32_t gC1[2 * kGateRows];
__shared__ __attribute__((aligned(16))) uint32_t gC3[2 * kGateRows];

// One 16- or 4-byte copy per lane, global -> LDS (M0 = the wave's LDS base;
// lane l's bytes land at base + size * l). Issued as inline assembly so that
// the compiler neither waits on it nor counts it; the kernel waits with
// explicit s_waitcnt vmcnt. Each statement names M0 as clobbered, so the
// compiler keeps no value of its own in M0 across it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)p);
}
// M0 is a register the compiler reserves: it never allocates it, but sets it
// right before its own instructions that read it. Naming it clobbered orders
// these statements against such uses; the compiler still warns that it does
// not preserve reserved registers, which is what is wanted here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (one VGPR per copy instead of a 64-bit address pair).
__device__ __forceinline__ void dma16s(uint32_t off, const void* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4s(uint32_t off, const void* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS stage layouts. A: 128 rows x 64 bf16 (128 B, 8 pieces of 16 B), piece
// p of row r at position p ^ ((r >> 1) & 7). B: 256 rows (gate 0..127, up
// 128..255) x 64 codes (64 B, 4 pieces), piece p at p ^ ((r >> 2) & 3).
// (The maps are involutions: position -> piece is the same formula.)
__device__ __forceinline__ int a_pos(int row, int piece) { return piece ^ ((row >> 1) & 7); }
__device__ __forceinline__ int b_pos(int row, int piece) { return piece ^ ((row >> 2) & 3); }

template <WFmt F, typename AT>
__global__ void __launch_bounds__(kGThreads)
k_gateup_gemm(const uint16_t* __restrict__ xa, const float* __restrict__ sx, int K,
              const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int E, int N, int k,
              const int32_t* __restrict__ expert_off, const int32_t* __restrict__ sorted_pairs,
              float* __restrict__ gu, AT* __restrict__ act, int ntiles) {
  // unit: the units of expert e run on XCD e % 8, consecutive in dispatch order
  const int blk = blockIdx.x;
  const int slot = blk / kXcds;
  const int e = (blk % kXcds) + kXcds * (slot / ntiles);
  const int nt = slot % ntiles;
  if (e >= E) return;
  const int r0 = expert_off[e];
  const int m_e = expert_off[e + 1] - r0;
  if (m_e <= 0) return;

  const int I = N / 2, G = K / kGroup, NB = N / kGroup;
  const int S = 2 * G;                           // stages per pass
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: kept in a scalar register
  const int col = lane % 32, half = lane / 32;
  const int ns = wave % 4;                       // column slice of this wave
  const int i0 = nt * kGateRows + 32 * ns;
  const int mw = 64 * (wave / 4);                // first pass row of this wave
  const bool live = i0 < I;                      // I % 32 == 0: a live wave has all 32 rows
  const int rg = 32 * ns + col, ru = kGateRows + 32 * ns + col;  // this lane's code rows in a B stage
  // LDS byte addresses of the ring (scalar, computed once)
  const uint32_t la0 = lds_addr(gA0), la1 = lds_addr(gA1), la2 = lds_addr(gA2), la3 = lds_addr(gA3);
  const uint32_t lb0 = lds_addr(gB0), lb1 = lds_addr(gB1), lb2 = lds_addr(gB2), lb3 = lds_addr(gB3);
  const uint32_t lc1 = lds_addr(gC1), lc3 = lds_addr(gC3);

  // code rows this lane copies: instruction q fills B rows 16 (2 wave + q) ..
  // +15; lane l takes row R + l / 4 and LDS position l % 4. Rows past I
  // repeat row 0 of the expert (never used).
  size_t bsrc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 16 * (2 * wave + q) + lane / 4;
    const int gi = nt * kGateRows + (row % kGateRows);
    const int n = gi < I ? (row < kGateRows ? gi : I + gi) : 0;
    bsrc[q] = ((size_t)e * N + n) * K + 16 * b_pos(row, lane % 4);
  }
  // side data copied by this lane with the odd stage of group g (dword of
  // element index base + g; the wanted bf16 is its half (base + g) & 1):
  //   int8, waves 0..3: the scale of code row 64 wave + lane of the unit
  //   E4M3, wave 2: block scale (lane % 2: gate, up) of column slice lane / 2 % 4
  int64_t cbase = 0;  // element index at group 0
  if constexpr (F == WFmt::I8) {
    const int row = 64 * (wave & 3) + lane;
    const int gi = nt * kGateRows + (row % kGateRows);
    const int n = gi < I ? (row < kGateRows ? gi : I + gi) : 0;
    cbase = ((int64_t)e * N + n) * G;
  } else {
    const int sl = (lane / 2) % 4, up = lane % 2;
    const int gi = nt * kGateRows + 32 * sl;
    const int nb = gi < I ? (up ? (I + gi) / kGroup : gi / kGroup) : 0;
    cbase = ((int64_t)e * NB + nb) * G;
  }
  // parity of the element index (at group 0) of the scales this lane reads
  // back in the fold: which half of the copied dword holds the bf16
  int par_g, par_u;
  if constexpr (F == WFmt::I8) {
    par_g = (int)((((int64_t)e * N + (live ? i0 + col : 0)) * G) & 1);
    par_u = (int)((((int64_t)e * N + (live ? I + i0 + col : 0)) * G) & 1);
  } else {
    par_g = (int)((((int64_t)e * NB + (live ? i0 / kGroup : 0)) * G) & 1);
    par_u = (int)((((int64_t)e * NB + (live ? (I + i0) / kGroup : 0)) * G) & 1);
  }

  for (int mb = 0; mb < m_e; mb += kPassRows) {
    const int rows = min(kPassRows, m_e - mb);
    const bool busy = live && rows > mw;         // the wave has live rows in this pass
    // activation rows this lane copies: instruction q fills A rows
    // 8 (2 wave + q) .. +7; lane l takes row R + l / 8 and LDS position l % 8.
    // Rows past the pass repeat the last valid row (their results are never stored).
    int asrc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = 8 * (2 * wave + q) + lane / 8;
      const int t = sorted_pairs[r0 + mb + min(row, rows - 1)] / k;
      asrc[q] = t * K + 8 * a_pos(row, lane % 8);
    }
    int xrow_tok = 0;                            // E4M3, waves 0, 1: token of pass row 64 wave + lane
    if constexpr (F == WFmt::E4M3) {
      const int row = 64 * (wave & 1) + lane;
      xrow_tok = sorted_pairs[r0 + mb + min(row, rows - 1)] / k;
    }

    // stage h = (group h / 2, K half h % 2) into the given ring slot (LDS byte
    // addresses of its A, B and side arrays); the odd stage of a group also
    // brings the group's side data
    auto issue = [&](int h, uint32_t aslot, uint32_t bslot, uint32_t cslot) {
      const int koff = h * kStageK;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        dma16(xa + asrc[q] + koff, aslot + (2 * wave + q) * (8 * kStageK * 2));
        dma16(codes + bsrc[q] + koff, bslot + (2 * wave + q) * (16 * kStageK));
      }
      if (h & 1) {
        const int g = h / 2;
        if constexpr (F == WFmt::I8) {
          if (wave < 4) dma4(scales + ((cbase + g) & ~(int64_t)1), cslot + 64 * 4 * wave);
        } else {
          if (wave < 2) dma4(sx + (size_t)xrow_tok * G + g, cslot + 64 * 4 * wave);
          else if (wave == 2) dma4(scales + ((cbase + g) & ~(int64_t)1), cslot + 4 * kGateRows);
        }
      }
    };

    f32x16 acc[kMTiles][2], tmp[kMTiles][2];
#pragma unroll
    for (int a = 0; a < kMTiles; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          acc[a][c][j] = 0.0f;
          tmp[a][c][j] = 0.0f;
        }

    auto half_bf16 = [](uint32_t w, int odd) { return __uint_as_float(odd ? (w & 0xffff0000u) : (w << 16)); };

    auto stage = [&](int h, const uint16_t* abuf, const uint8_t* bbuf, const uint32_t* cbuf,
                     uint32_t anext, uint32_t bnext, uint32_t cnext) {
      if (h >= S) return;
      const int g = h / 2, hh = h % 2;
      // wait for this wave's copies of stage h: the copies of the stages issued
      // after it (4 each, plus side data) may stay in flight
      const int later = min(2, S - 1 - h);
      if (later == 2) __builtin_amdgcn_s_waitcnt(wait_vm(8));
      else if (later == 1) __builtin_amdgcn_s_waitcnt(wait_vm(4));
      else __builtin_amdgcn_s_waitcnt(wait_vm(0));
      __builtin_amdgcn_s_barrier();            // ... and every other wave's
      if (h + 3 < S) issue(h + 3, anext, bnext, cnext);  // the slot of stage h - 1, now free
      if (!busy) return;
      if (hh == 0) {
#pragma unroll
        for (int a = 0; a < kMTiles; ++a)
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 16; ++j) tmp[a][c][j] = 0.0f;
      }
      // the lane's 32 codes of the stage (k = 32 half .. +31) are pieces
      // 2 half and 2 half + 1 of its gate and up rows: piece q serves k-steps
      // 2 q and 2 q + 1
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 cg, cu;
        cg = *reinterpret_cast<const u32x4*>(&bbuf[rg * kStageK + 16 * b_pos(rg, 2 * half + s / 2)]);
        cu = *reinterpret_cast<const u32x4*>(&bbuf[ru * kStageK + 16 * b_pos(ru, 2 * half + s / 2)]);
        const bf16x8 wg = decode8<F>(cg[2 * (s % 2)], cg[2 * (s % 2) + 1]);
        const bf16x8 wu = decode8<F>(cu[2 * (s % 2)], cu[2 * (s % 2) + 1]);
#pragma unroll
        for (int a = 0; a < kMTiles; ++a) {
          const int m = mw + 32 * a + col;
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(&abuf[m * kStageK + 8 * a_pos(m, 4 * half + s)]);
          tmp[a][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, wg, tmp[a][0], 0, 0, 0);
          tmp[a][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, wu, tmp[a][1], 0, 0, 0);
        }
      }
      if (hh == 1) {
        if constexpr (F == WFmt::I8) {
          const float sg = half_bf16(cbuf[rg], (par_g + g) & 1), su = half_bf16(cbuf[ru], (par_u + g) & 1);
#pragma unroll
          for (int a = 0; a < kMTiles; ++a)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              acc[a][0][j] = fmaf(tmp[a][0][j], sg, acc[a][0][j]);
              acc[a][1][j] = fmaf(tmp[a][1][j], su, acc[a][1][j]);
            }
        } else {
          const float wg = half_bf16(cbuf[kGateRows + 2 * ns], (par_g + g) & 1);
          const float wu = half_bf16(cbuf[kGateRows + 2 * ns + 1], (par_u + g) & 1);
#pragma unroll
          for (int a = 0; a < kMTiles; ++a)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const float f = __uint_as_float(cbuf[mw + 32 * a + 8 * (j / 4) + 4 * half + (j % 4)]);
              acc[a][0][j] = fmaf(tmp[a][0][j], wg * f, acc[a][0][j]);
              acc[a][1][j] = fmaf(tmp[a][1][j], wu * f, acc[a][1][j]);
            }
        }
      }
    };

    __builtin_amdgcn_s_barrier();  // nobody still reads the ring of the previous pass
    issue(0, la0, lb0, 0);
    if (S > 1) issue(1, la1, lb1, lc1);
    if (S > 2) issue(2, la2, lb2, 0);
    for (int hb = 0; hb < S; hb += kSlots) {     // stage h uses slot h % 4, fixed at compile time
      stage(hb + 0, gA0, gB0, nullptr, la3, lb3, lc3);
      stage(hb + 1, gA1, gB1, gC1, la0, lb0, 0);
      stage(hb + 2, gA2, gB2, nullptr, la1, lb1, lc1);
      stage(hb + 3, gA3, gB3, gC3, la2, lb2, 0);
    }
    if (busy) {
#pragma unroll
      for (int a = 0; a < kMTiles; ++a) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int m = mw + 32 * a + 8 * (j / 4) + 4 * half + (j % 4);
          if (m < rows) {
            const size_t r = (size_t)(r0 + mb + m);
            const float gv = acc[a][0][j], uv = acc[a][1][j];
            if (gu) {
              gu[r * N + i0 + col] = gv;
              gu[r * N + I + i0 + col] = uv;
            }
            if (act) put_act(act, r * I + i0 + col, gelu_tanh(gv) * uv);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// int8, tall passes: 256 pairs x 128 gate (+128 up) columns per unit and pass.
//
// The result is kept in units of the current group's scale: for column n,
//   R = (sum over groups so far of s_g * P_g) / s_current,
// so a new group only multiplies R by s_current / s_new (one multiply per
// element, no second accumulator) and the MFMAs add that group's plain code
// products P_g on top; the stored value is R * s_last. The ratio adds about
// two float32 roundings per group. A zero scale keeps the current one and its
// codes are masked to zero, so such a group contributes exactly nothing. So
// does a group whose scale lies more than 2^64 below the largest one taken
// before it in the row: that keeps |R| below 2^64 * 127 * K * max|x|, finite
// for any activation below 2^46 at K = 2048 (a dropped group's terms are
// below 2^-64 s_max 127 sum|x|; terms more than 2^126 below a later, larger
// scale underflow the same way).
// Freed of the second accumulator, each wave holds 4 m-tiles x (32 gate + 32
// up) columns: every code it decodes feeds four MFMAs, and a prefill-sized
// expert (up to 256 pairs) is covered in one pass, so its codes are read
// once.
//
// Waves: wm = wave / 4 takes the m-tiles (32 pass rows each) 2a + wm, a < 4,
// interleaved so that both waves sharing a SIMD have work when an expert
// has about 128 pairs; wn = wave % 4 takes the gate columns 32 wn .. +31 of
// the unit and the matching up columns. A wave with no live m-tile skips the
// products (NA = 0), one with at most two computes two, else three or four.
// Ring: 3 slots (A 32 KB, B 16 KB, scales 2 KB each), two stages in flight
// while one is multiplied. Group 0's scales come with stage 0, group g + 1's
// with the last stage of group g, where each m-tile is rescaled right after
// its last product of the group (so the multiplies overlap the products of
// the other tiles instead of starting the next group on their own).
constexpr int kTThreads = 512;
constexpr int kTRows = 256;
constexpr int kTGate = 128;

__shared__ __attribute__((aligned(16))) uint16_t tA0[kTRows * kStageK];
__shared__ __attribute__((aligned(16))) uint16_t tA1[kTRows * kStageK];
__shared__ __attribute__((aligned(16))) uint16_t tA2[kTRows * kStageK];
__shared__ __attribute__((aligned(16))) uint8_t tB0[2 * kTGate * kStageK];
__shared__ __attribute__((aligned(16))) uint8_t tB1[2 * kTGate * kStageK];
__shared__ __attribute__((aligned(16))) uint8_t tB2[2 * kTGate * kStageK];
// scales of the unit's 256 code rows for one group: B row r at 64 (r / 32) + r % 32
__shared__ __attribute__((aligned(16))) uint32_t tC0[2 * kTRows];
__shared__ __attribute__((aligned(16))) uint32_t tC1[2 * kTRows];
__shared__ __attribute__((aligned(16))) uint32_t tC2[2 * kTRows];

// Stage layouts, bank-conflict free for 16-byte reads by 16 consecutive
// lanes (consecutive rows) over the 64 four-byte banks: A piece p (8 bf16)
// of row r (128 bytes) at p ^ ((r >> 1) & 7); B piece p (16 codes) of row r
// (64 bytes) at p ^ ((r >> 2) & 3). Within a 64-K stage, MFMA k-step s takes
// k = 32 h + 8 s .. +7 in the lanes of half h, so a B lane reads one
// contiguous 32-byte span (pieces 2h, 2h+1) and an A lane piece 4h + s; both
// sides agree on every k.
__device__ __forceinline__ int ta_pos(int row, int piece) { return piece ^ ((row >> 1) & 7); }
__device__ __forceinline__ int tb_pos(int row, int piece) { return piece ^ ((row >> 2) & 3); }

// s_waitcnt vmcnt(n) for a count known only at run time (uniform, 0..8)
__device__ __forceinline__ void wait_vm_dyn(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(wait_vm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(wait_vm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(wait_vm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(wait_vm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(wait_vm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(wait_vm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(wait_vm(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(wait_vm(7)); break;
    default: __builtin_amdgcn_s_waitcnt(wait_vm(8)); break;
  }
}

template <int NA>
struct TallPass {
  f32x16 R[4][2];
};

template <typename AT>
__global__ void __launch_bounds__(kTThreads)
k_gateup_gemm_tall(const uint16_t* __restrict__ xa, int K, const uint8_t* __restrict__ codes,
                   const uint16_t* __restrict__ scales, int E, int N, int k,
                   const int32_t* __restrict__ expert_off, const int32_t* __restrict__ sorted_pairs,
                   float* __restrict__ gu, AT* __restrict__ act, int ntiles) {
  const int blk = blockIdx.x;
  const int slot = blk / kXcds;
  const int e = (blk % kXcds) + kXcds * (slot / ntiles);
  const int nt = slot % ntiles;
  if (e >= E) return;
  const int r0 = expert_off[e];
  const int m_e = expert_off[e + 1] - r0;
  if (m_e <= 0) return;

  const int I = N / 2, G = K / kGroup;
  const int S = 2 * G;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane % 32, half = lane / 32;
  const int wm = wave / 4, wn = wave % 4;
  const int i0 = nt * kTGate + 32 * wn;
  const bool live = i0 < I;
  const int rg = 32 * wn + col, ru = kTGate + 32 * wn + col;  // this lane's code rows in a B stage
  const uint32_t la0 = lds_addr(tA0), la1 = lds_addr(tA1), la2 = lds_addr(tA2);
  const uint32_t lb0 = lds_addr(tB0), lb1 = lds_addr(tB1), lb2 = lds_addr(tB2);
  const uint32_t lc0 = lds_addr(tC0), lc1 = lds_addr(tC1), lc2 = lds_addr(tC2);

  // copies use per-block bases (SGPRs) and 32-bit byte offsets (N K < 2^31)
  const uint8_t* cbase_p = codes + (size_t)e * N * K;
  const int64_t sidx0 = ((int64_t)e * N * G) & ~(int64_t)1;         // dword-aligned first scale of e
  const uint16_t* sbase_p = scales + sidx0;
  // code rows this lane copies (instruction q: B rows 16 (2 wave + q) .. +15)
  uint32_t boff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 16 * (2 * wave + q) + lane / 4;
    const int gi = nt * kTGate + (row % kTGate);
    const int n = gi < I ? (row < kTGate ? gi : I + gi) : 0;
    boff[q] = (uint32_t)n * (uint32_t)K + 16 * tb_pos(row, lane % 4);
  }
  // scale dword this lane copies: B row 32 wave + lane % 32 (lanes 32..63 repeat it);
  // coff = element index of its group-0 scale relative to sidx0
  uint32_t coff;
  {
    const int row = 32 * wave + (lane % 32);
    const int gi = nt * kTGate + (row % kTGate);
    const int n = gi < I ? (row < kTGate ? gi : I + gi) : 0;
    coff = (uint32_t)(((int64_t)e * N + n) * G - sidx0);
  }
  const int par_g = (int)((((int64_t)e * N + (live ? i0 + col : 0)) * G) & 1);
  const int par_u = (int)((((int64_t)e * N + (live ? I + i0 + col : 0)) * G) & 1);
  const int cg_idx = 64 * (rg / 32) + (rg % 32), cu_idx = 64 * (ru / 32) + (ru % 32);
  // LDS read offsets (bytes). The swizzles do not depend on the m-tile or on
  // gate/up (rows 128 wm + 32 a + col and 32 wn + col (+128) share their low
  // bits with col), so one base per A k-step and per B piece; m-tile (4096 a
  // bytes) and up (8192 bytes) are immediates.
  uint32_t aoffs[4], boffs[2];
#pragma unroll
  for (int st = 0; st < 4; ++st)
    aoffs[st] = (uint32_t)((32 * wm + col) * (kStageK * 2) + 16 * ((4 * half + st) ^ ((col >> 1) & 7)));
#pragma unroll
  for (int pc = 0; pc < 2; ++pc) boffs[pc] = (uint32_t)(rg * kStageK + 16 * ((2 * half + pc) ^ ((col >> 2) & 3)));
  auto half_bf16 = [](uint32_t w, int odd) { return __uint_as_float(odd ? (w & 0xffff0000u) : (w << 16)); };

  for (int mb = 0; mb < m_e; mb += kTRows) {
    const int rows = min(kTRows, m_e - mb);
    const int mtiles = (rows + 31) / 32;                   // live m-tiles of the pass
    const int na = live && mtiles > wm ? min(4, (mtiles - wm + 1) / 2) : 0;
    // this wave copies A rows 32 wave .. +31 in four 8-row copies: only those
    // holding pass rows (rows past the pass are never stored)
    const int nca = min(4, max(0, (rows - 32 * wave + 7) / 8));
    uint32_t aoff[4];  // byte offsets into x_rot
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 8 * (4 * wave + q) + lane / 8;
      const int t = sorted_pairs[r0 + mb + min(row, rows - 1)] / k;
      aoff[q] = 2u * ((uint32_t)t * (uint32_t)K + 8 * ta_pos(row, lane % 8));
    }
    // stages that bring scales: 0 (group 0) and 2g + 1 (group g + 1, if any)
    auto has_c = [&](int h) { return h == 0 || ((h & 1) && (h + 1) / 2 < G); };
    // copies per stage of this wave: A, 2 B, and the scales
    auto dmas = [&](int h) { return nca + 2 + (has_c(h) ? 1 : 0); };

    auto issue = [&](int h, uint32_t aslot, uint32_t bslot, uint32_t cslot) __attribute__((always_inline)) {
      const uint32_t koff = (uint32_t)h * kStageK;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q < nca) dma16s(aoff[q] + 2u * koff, xa, aslot + (4 * wave + q) * (8 * kStageK * 2));
#pragma unroll
      for (int q = 0; q < 2; ++q) dma16s(boff[q] + koff, cbase_p, bslot + (2 * wave + q) * (16 * kStageK));
      if (has_c(h)) dma4s(2u * ((coff + (h + 1) / 2) & ~1u), sbase_p, cslot + 4 * kWave * wave);
    };

    f32x16 R[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) R[a][c][j] = 0.0f;
    float seff_g = 1.0f, seff_u = 1.0f;  // the scale R is currently expressed in
    float smax_g = 0.0f, smax_u = 0.0f;  // largest scale taken so far; 0 while R is still exactly 0
    uint32_t mask_g = ~0u, mask_u = ~0u;
    bool need_mask = false;
    // A group's scale s joins the running result unless it is zero or lies
    // more than 2^64 below the largest scale taken before it in the row
    // (then the group is masked like a zero-scale one: its terms are below
    // 2^-64 of that scale's). This bounds every rescale factor by 2^64, so R
    // stays finite; nothing is rescaled while R is still exactly 0.
    auto take = [](float sc, float smax) { return sc != 0.0f && sc >= smax * 0x1p-64f; };

    auto body = [&](auto na_c, int h, const uint16_t* abuf, const uint8_t* bbuf, const uint32_t* cbuf)
        __attribute__((always_inline)) {
      constexpr int NA = decltype(na_c)::value;
      // scales of the group that starts next (read before this stage's products)
      const bool next_c = (h & 1) && (h + 1) / 2 < G;
      float sg = 0.0f, su = 0.0f;
      if (h == 0 || next_c) {
        const int g = (h + 1) / 2;
        sg = half_bf16(cbuf[cg_idx], (par_g + g) & 1);
        su = half_bf16(cbuf[cu_idx], (par_u + g) & 1);
      }
      if (h == 0) {
        const bool tg = sg != 0.0f, tu = su != 0.0f;
        if (tg) seff_g = smax_g = sg;
        if (tu) seff_u = smax_u = su;
        mask_g = tg ? ~0u : 0u;
        mask_u = tu ? ~0u : 0u;
        need_mask = __ballot(!tg || !tu) != 0;
      }
      u32x4 cgp[2], cup[2];  // the lane's 32 codes of its gate and up rows in this stage
#pragma unroll
      for (int pc = 0; pc < 2; ++pc) {
        cgp[pc] = *reinterpret_cast<const u32x4*>(bbuf + boffs[pc]);
        cup[pc] = *reinterpret_cast<const u32x4*>(bbuf + boffs[pc] + kTGate * kStageK);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4& cg4 = cgp[s / 2];
        const u32x4& cu4 = cup[s / 2];
        bf16x8 wg = decode8<WFmt::I8>(cg4[2 * (s % 2)], cg4[2 * (s % 2) + 1]);
        bf16x8 wu = decode8<WFmt::I8>(cu4[2 * (s % 2)], cu4[2 * (s % 2) + 1]);
        if (need_mask) {
          u32x4 mg = __builtin_bit_cast(u32x4, wg), mu = __builtin_bit_cast(u32x4, wu);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            mg[w] &= mask_g;
            mu[w] &= mask_u;
          }
          wg = __builtin_bit_cast(bf16x8, mg);
          wu = __builtin_bit_cast(bf16x8, mu);
        }
#pragma unroll
        for (int a = 0; a < NA; ++a) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint8_t*>(abuf) + aoffs[s] +
                                                             64 * a * (kStageK * 2));
          R[a][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, wg, R[a][0], 0, 0, 0);
          R[a][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, wu, R[a][1], 0, 0, 0);
        }
      }
      if (next_c) {
        // express R in the next group's scale; a masked group keeps the
        // current one (factors within [2^-64, 2^64] once R holds a term)
        const bool tg = take(sg, smax_g), tu = take(su, smax_u);
        const float rgt = tg && smax_g != 0.0f ? seff_g / sg : 1.0f;
        const float rut = tu && smax_u != 0.0f ? seff_u / su : 1.0f;
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            R[a][0][j] *= rgt;
            R[a][1][j] *= rut;
          }
        if (tg) {
          seff_g = sg;
          smax_g = fmaxf(smax_g, sg);
        }
        if (tu) {
          seff_u = su;
          smax_u = fmaxf(smax_u, su);
        }
        mask_g = tg ? ~0u : 0u;
        mask_u = tu ? ~0u : 0u;
        need_mask = __ballot(!tg || !tu) != 0;
      }
    };

    auto stage = [&](auto na_c, int h, const uint16_t* abuf, const uint8_t* bbuf, const uint32_t* cbuf,
                     uint32_t anext, uint32_t bnext, uint32_t cnext) __attribute__((always_inline)) {
      if (h >= S) return;
      // wait for this wave's copies of stage h (those of stage h + 1 may stay in flight)
      wait_vm_dyn(h + 1 < S ? dmas(h + 1) : 0);
      __builtin_amdgcn_s_barrier();            // ... and every other wave's
      if (h + 2 < S) issue(h + 2, anext, bnext, cnext);  // the slot of stage h - 1, now free
      constexpr int NA = decltype(na_c)::value;
      if constexpr (NA > 0) body(na_c, h, abuf, bbuf, cbuf);
    };

    auto run = [&](auto na_c) __attribute__((always_inline)) {
      __builtin_amdgcn_s_barrier();  // nobody still reads the ring of the previous pass
      issue(0, la0, lb0, lc0);
      if (S > 1) issue(1, la1, lb1, lc1);
      for (int hb = 0; hb < S; hb += 3) {       // stage h uses slot h % 3, fixed at compile time
        stage(na_c, hb + 0, tA0, tB0, tC0, la2, lb2, lc2);
        stage(na_c, hb + 1, tA1, tB1, tC1, la0, lb0, lc0);
        stage(na_c, hb + 2, tA2, tB2, tC2, la1, lb1, lc1);
      }
    };
    if (na > 3) run(std::integral_constant<int, 4>{});
    else if (na > 2) run(std::integral_constant<int, 3>{});
    else if (na > 0) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 0>{});

    if (na > 0) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if (a >= na) break;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int m = 32 * (2 * a + wm) + 8 * (j / 4) + 4 * half + (j % 4);
          if (m < rows) {
            const size_t r = (size_t)(r0 + mb + m);
            const float gv = R[a][0][j] * seff_g, uv = R[a][1][j] * seff_u;
            if (gu) {
              gu[r * N + i0 + col] = gv;
              gu[r * N + I + i0 + col] = uv;
            }
            if (act) put_act(act, r * I + i0 + col, gelu_tanh(gv) * uv);
          }
        }
      }
    }
  }
}

static int gemm_grid(int E, int ntiles) { return cdiv(E, kXcds) * kXcds * ntiles; }

hipError_t launch_gateup_i8h_gemm_tall(const uint16_t* xrot, int T, int K, const int8_t* codes,
                                       const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                       const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16,
                                       hipStream_t st) {
  (void)T;
  int ntiles = cdiv(N / 2, kTGate);
  const uint8_t* q = reinterpret_cast<const uint8_t*>(codes);
  if (act_bf16)
    k_gateup_gemm_tall<<<gemm_grid(E, ntiles), kTThreads, 0, st>>>(xrot, K, q, scales, E, N, k, expert_off,
                                                                   sorted_pairs, gu,
                                                                   static_cast<uint16_t*>(act), ntiles);
  else
    k_gateup_gemm_tall<<<gemm_grid(E, ntiles), kTThreads, 0, st>>>(xrot, K, q, scales, E, N, k, expert_off,
                                                                   sorted_pairs, gu, static_cast<float*>(act),
                                                                   ntiles);
  return hipGetLastError();
}

template <WFmt F>
static hipError_t launch_gemm(const uint16_t* xa, const float* sx, int K, const uint8_t* codes,
                              const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                              const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16, hipStream_t st) {
  const int ntiles = cdiv(N / 2, kGateRows);
  if (act_bf16)
    k_gateup_gemm<F><<<gemm_grid(E, ntiles), kGThreads, 0, st>>>(xa, sx, K, codes, scales, E, N, k, expert_off,
                                                                 sorted_pairs, gu, static_cast<uint16_t*>(act),
                                                                 ntiles);
  else
    k_gateup_gemm<F><<<gemm_grid(E, ntiles), kGThreads, 0, st>>>(xa, sx, K, codes, scales, E, N, k, expert_off,
                                                                 sorted_pairs, gu, static_cast<float*>(act),
                                                                 ntiles);
  return hipGetLastError();
}

hipError_t launch_gateup_i8h_gemm(const uint16_t* xrot, int T, int K, const int8_t* codes,
                                  const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                  const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16,
                                  hipStream_t st) {
  (void)T;
  return launch_gemm<WFmt::I8>(xrot, nullptr, K, reinterpret_cast<const uint8_t*>(codes), scales, E, N, k,
                               expert_off, sorted_pairs, gu, act, act_bf16, st);
}

hipError_t launch_gateup_fp8(const uint16_t* xq, const float* sx, int T, int K, const uint8_t* codes,
                             const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                             const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16, hipStream_t st) {
  (void)T;
  return launch_gemm<WFmt::E4M3>(xq, sx, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu, act, act_bf16,
                                 st);
}

}  // namespace i8h
