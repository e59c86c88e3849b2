// bf16 grouped down projection of the routed experts and the weighted combine
// of each token's k expert outputs: the step after the gate_up path.
//
// The int8 card's model table (row "Weights") keeps the experts' down
// projections in bf16. W_down[e] is [H, I] row-major (H = the hidden size);
// the float32 act rows of the gate_up epilogue are rounded to bf16 (nearest
// even) for the product, or come already rounded (the gate_up epilogue's bf16
// form, AT = uint16_t), and it accumulates in float32 (products of two bf16
// values are exact in float32; the few-pairs form adds them two at a time
// with v_dot2_f32_bf16):
//   y[r, h]   = sum_i W_down[e(r), h, i] * bf16(act[r, i])      (sorted row r)
//   out[t, h] = sum_j w[t, j] * y[pos[t k + j], h]              (slot order j)
//
// Two forms:
//   * few pairs (decode): one kernel computes out directly. A workgroup owns
//     8 output rows h of one token and every slot j of it: each half-wave
//     streams the 8 rows of one expert with 16-byte loads and dots them with
//     the token's act row for that slot; the 8 x k partial dots meet in LDS
//     and are merged in slot order. No intermediate y, one launch.
//   * many pairs (verify, prefill): act -> bf16 once (nothing to do for bf16
//     act), a grouped bf16 MFMA GEMM
//     writes y in sorted order, then a combine kernel merges the k rows of
//     each token. The GEMM is persistent: a workgroup per CU streams work
//     items (expert, 256 output columns), each in passes of 256 sorted rows,
//     back to back; 64-byte-per-row stages of A (act rows) and B (W_down rows)
//     go global -> LDS by gfx950's DMA into a 4-slot ring, and eight waves
//     (two per SIMD) each hold 4 m-tiles x 2 column tiles of
//     v_mfma_f32_32x32x16_bf16 results.

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

namespace i8h {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

// ---------------------------------------------------------------------------
// Few pairs: out[t, h0 .. h0 + 7] of one token per workgroup.

constexpr int kDvRows = 8;       // output rows per workgroup

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// c + a.lo * b.lo + a.hi * b.hi for two pairs of bf16 values (v_dot2_f32_bf16:
// one instruction per two products, on the packed pairs as loaded)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}
constexpr int kDvThreads = 256;  // 8 half-waves

// NQ: 16-byte pieces (8 bf16) per lane per row, I <= 256 * NQ
template <int NQ, typename AT>
__global__ void __launch_bounds__(kDvThreads)
k_down_gemv_combine(const AT* __restrict__ act, int I, const uint16_t* __restrict__ w, int H, int k,
                    const int32_t* __restrict__ ids, const float* __restrict__ tw,
                    const int32_t* __restrict__ pos, float* __restrict__ out) {
  __shared__ float part[kMaxTopk][kDvRows];
  const int t = blockIdx.y, h0 = blockIdx.x * kDvRows;
  const int tid = threadIdx.x, hw = tid / 32, l = tid % 32;
  const int npc = I / 8;  // 16-byte pieces per row
  for (int j = hw; j < k; j += kDvThreads / 32) {
    const int e = ids[t * k + j];
    const int r = pos[t * k + j];
    // the 8 weight rows first (their loads are the stream), then the act row
    const uint16_t* wr = w + ((size_t)e * H + h0) * I;
    u32x4 wv[kDvRows][NQ];
#pragma unroll
    for (int row = 0; row < kDvRows; ++row)
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        // a piece past the row re-reads the last one (finite; its act pair is zero)
        const int c = min(l + 32 * q, npc - 1);
        wv[row][q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr + (size_t)row * I + 8 * c));
      }
    // the act values rounded to bf16 (nearest even), in pairs as the weights are
    uint32_t a[NQ][4];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int c = l + 32 * q;
      if constexpr (std::is_same_v<AT, float>) {
        f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
        if (c < npc) {
          lo = *reinterpret_cast<const f32x4*>(act + (size_t)r * I + 8 * c);
          hi = *reinterpret_cast<const f32x4*>(act + (size_t)r * I + 8 * c + 4);
        }
        a[q][0] = pack_bf16x2(lo[0], lo[1]);
        a[q][1] = pack_bf16x2(lo[2], lo[3]);
        a[q][2] = pack_bf16x2(hi[0], hi[1]);
        a[q][3] = pack_bf16x2(hi[2], hi[3]);
      } else {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (c < npc) v = *reinterpret_cast<const u32x4*>(act + (size_t)r * I + 8 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[q][i] = v[i];
      }
    }
#pragma unroll
    for (int row = 0; row < kDvRows; ++row) {
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) s = dot2_bf16(wv[row][q][i], a[q][i], s);
      s += xor_lane<1>(s);
      s += xor_lane<2>(s);
      s += xor_lane<4>(s);
      s += xor_lane<8>(s);
      s += xor_lane<16>(s);
      if (l == 0) part[j][row] = s;
    }
  }
  __syncthreads();
  if (tid < kDvRows) {
    float o = 0.0f;
    for (int j = 0; j < k; ++j) o = fmaf(tw[t * k + j], part[j][tid], o);
    out[(size_t)t * H + h0 + tid] = o;
  }
}

// ---------------------------------------------------------------------------
// Many pairs: act -> bf16, grouped GEMM into y, combine.

__global__ void k_f32_to_bf16(const float* __restrict__ src, uint16_t* __restrict__ dst, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4 lo = reinterpret_cast<const f32x4*>(src)[2 * i];
  const f32x4 hi = reinterpret_cast<const f32x4*>(src)[2 * i + 1];
  u32x4 o;
  o[0] = pack_bf16x2(lo[0], lo[1]);
  o[1] = pack_bf16x2(lo[2], lo[3]);
  o[2] = pack_bf16x2(hi[0], hi[1]);
  o[3] = pack_bf16x2(hi[2], hi[3]);
  reinterpret_cast<u32x4*>(dst)[i] = o;
}

constexpr int kDgThreads = 512;              // 8 waves, two per SIMD
constexpr int kDgRows = 256;                 // sorted rows per pass
constexpr int kDgCols = 256;                 // output columns per unit
constexpr int kDgStageK = 32;                // bf16 per row per stage (64 bytes)
constexpr int kDgSlots = 4;
constexpr int kDgASlot = kDgRows * kDgStageK * 2;   // 16 KB
constexpr int kDgBSlot = kDgCols * kDgStageK * 2;   // 16 KB
constexpr int kDgSlotBytes = kDgASlot + kDgBSlot;
constexpr int kDgXcds = 8;
constexpr int kDgBlocks = 256;               // one resident workgroup per CU

__shared__ __attribute__((aligned(16))) uint8_t dRing[kDgSlots * kDgSlotBytes];

constexpr int dg_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// 16 bytes per lane global -> LDS (M0 = the wave's LDS base, lane l's bytes at
// base + 16 l), with a wave-uniform 64-bit base and a 32-bit lane offset. The
// compiler neither counts nor waits on it; the kernel waits with vmcnt.
// The base goes through readfirstlane: it is uniform, but the compiler does not
// always prove it, and an "s" operand must be an SGPR.
// M0 is a register the compiler reserves: it never allocates it, but sets it
// right before its own instructions that read it. Naming it clobbered orders
// these statements against such uses; the compiler still warns that it does
// not preserve reserved registers, which is what is wanted here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dg_dma16(uint32_t off, const void* base, uint32_t lds) {
  // (readfirstlane returns a signed int: take both halves as uint32_t before
  // widening, or a low word with bit 31 set would sign-extend over the high one)
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t u = ((uint64_t)hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off),
               "s"(reinterpret_cast<const void*>(u)), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// A row (or B row) of a stage is 64 bytes = 4 pieces of 16; piece p of row r
// sits at position p ^ ((r >> 2) & 3), so 16 consecutive rows read at one
// piece hit 64 distinct banks. (An involution: position -> piece alike.)
__device__ __forceinline__ int dg_pos(int row, int piece) { return piece ^ ((row >> 2) & 3); }

// s_waitcnt vmcnt(n) for a wave-uniform n known at run time (0..8)
__device__ __forceinline__ void dg_wait_rt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(dg_vm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(dg_vm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(dg_vm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(dg_vm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(dg_vm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(dg_vm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(dg_vm(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(dg_vm(7)); break;
    default: __builtin_amdgcn_s_waitcnt(dg_vm(8)); break;
  }
}

__shared__ int32_t dEoff[kMaxExperts + 1];   // expert offsets, staged once

// One pass: up to 256 consecutive sorted rows of expert e against column tile nt.
struct DPass {
  int e, nt, r0, mb, rows;
};

// Persistent: a workgroup takes work items (expert e, column tile nt) b, b +
// grid, ... (the items of expert e on XCD e % 8, its column tiles on
// consecutive workgroups so they read its A rows from one L2), each one or
// more passes of 256 rows, and streams the passes' stages back to back: the
// next pass's first three stages are copied during the current pass's last
// three, and its y stores (which count in vmcnt) are issued after this wave
// has waited for the next pass's first stage, so nothing drains between
// passes. The A rows of a pass are contiguous (sorted order), so everything
// a pass needs comes from the staged offsets: no global load mid-stream.
__global__ void __launch_bounds__(kDgThreads)
k_down_gemm(const uint16_t* __restrict__ a16, int I, const uint16_t* __restrict__ w, int E, int H,
            const int32_t* __restrict__ expert_off, float* __restrict__ y, int ntiles) {
  const int S = I / kDgStageK;                 // stages per pass, at least 3
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 4, wn = wave % 4;     // m-tiles 2a + wm; columns 64 wn .. +63
  const int col = lane % 32, half = lane / 32;
  const uint32_t ring = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)dRing);
  const int nitems = cdiv(E, kDgXcds) * kDgXcds * ntiles;
  const int grid = gridDim.x;

  for (int i = tid; i <= E; i += kDgThreads) dEoff[i] = expert_off[i];
  __syncthreads();

  // B copies: instruction q fills W_down rows nt*256 + 16 (2 wave + q) + lane / 4
  // (the same offsets for every item, from the item's row base)
  uint32_t boff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 16 * (2 * wave + q) + lane / 4;
    boff[q] = (uint32_t)(row * I + 8 * dg_pos(row, lane % 4)) * 2u;
  }
  // fragment offsets within a slot: k-step s, lane half -> piece 2 s + half
  uint32_t aoffs[2], boffs[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    aoffs[s] = (uint32_t)(col * 64 + 16 * dg_pos(col, 2 * s + half));   // + 2048 per m-tile (rows 32 mt ..)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int n = 64 * wn + 32 * c + col;
      boffs[s][c] = (uint32_t)(kDgASlot + n * 64 + 16 * dg_pos(n, 2 * s + half));
    }
  }

  auto first_pass = [&](int& it, DPass& p) __attribute__((always_inline)) {
    for (; it < nitems; it += grid) {
      const int slot = it / kDgXcds;
      const int e = (it % kDgXcds) + kDgXcds * (slot / ntiles);
      if (e >= E) continue;
      const int r0 = dEoff[e], m = dEoff[e + 1] - r0;
      if (m <= 0) continue;
      p.e = __builtin_amdgcn_readfirstlane(e);
      p.nt = __builtin_amdgcn_readfirstlane(slot % ntiles);
      p.r0 = __builtin_amdgcn_readfirstlane(r0);
      p.mb = 0;
      p.rows = __builtin_amdgcn_readfirstlane(min(kDgRows, m));
      return true;
    }
    return false;
  };
  auto next_pass = [&](int& it, const DPass& c, DPass& p) __attribute__((always_inline)) {
    const int m = dEoff[c.e + 1] - c.r0;
    if (c.mb + kDgRows < m) {
      p = c;
      p.mb = c.mb + kDgRows;
      p.rows = __builtin_amdgcn_readfirstlane(min(kDgRows, m - p.mb));
      return true;
    }
    it += grid;
    return first_pass(it, p);
  };
  // A copies of this wave for a pass: instruction q fills pass rows
  // 16 (2 wave + q) + lane / 4, only blocks of 16 that hold pass rows (later
  // rows repeat the last one)
  auto a_src = [&](const DPass& p, uint32_t (&aoff)[2]) __attribute__((always_inline)) {
    int nca = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = 16 * (2 * wave + q) + lane / 4;
      if (16 * (2 * wave + q) < p.rows) ++nca;
      aoff[q] = (uint32_t)((p.r0 + p.mb + min(row, p.rows - 1)) * I + 8 * dg_pos(row, lane % 4)) * 2u;
    }
    return __builtin_amdgcn_readfirstlane(nca);
  };
  // stage hh of a pass into the slot of global stage g; returns this wave's copies
  auto issue = [&](const DPass& p, const uint32_t (&aoff)[2], int nca, int hh, int g)
      __attribute__((always_inline)) {
    const uint32_t sl = ring + (uint32_t)((g % kDgSlots) * kDgSlotBytes);
    const uint32_t koff = (uint32_t)hh * (kDgStageK * 2);
    const uint16_t* wbase = w + ((size_t)p.e * H + (size_t)p.nt * kDgCols) * I;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (q < nca) dg_dma16(aoff[q] + koff, a16, sl + (2 * wave + q) * 1024);
#pragma unroll
    for (int q = 0; q < 2; ++q) dg_dma16(boff[q] + koff, wbase, sl + kDgASlot + (2 * wave + q) * 1024);
    return nca + 2;
  };

  int item = blockIdx.x;
  DPass cur;
  if (!first_pass(item, cur)) return;
  uint32_t ca[2];
  int cn = a_src(cur, ca);
  // copies in flight are those of the stage waited for next and of the two
  // after it; c2 and c3 count the latter two
  issue(cur, ca, cn, 0, 0);
  int c2 = issue(cur, ca, cn, 1, 1), c3 = issue(cur, ca, cn, 2, 2);
  int g0 = 0;                   // global stage of the current pass's stage 0
  bool prewaited = false;

  while (true) {
    DPass nx;
    int item_n = item;
    const bool has_next = next_pass(item_n, cur, nx);
    uint32_t na_off[2] = {0u, 0u};
    int nn = 0;
    if (has_next) nn = a_src(nx, na_off);
    const int mtiles = (cur.rows + 31) / 32;
    const int na = (mtiles - wm + 1) / 2;     // live m-tiles 2a + wm of this wave

    auto run = [&](auto na_c) __attribute__((always_inline)) {
      constexpr int NA = decltype(na_c)::value;
      f32x16 R[NA > 0 ? NA : 1][2];
#pragma unroll
      for (int a = 0; a < (NA > 0 ? NA : 1); ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int j = 0; j < 16; ++j) R[a][c][j] = 0.0f;
      for (int hh = 0; hh < S; ++hh) {
        const int gs = g0 + hh;
        // this wave's copies of stage gs are in LDS (those of the two stages
        // after it may stay in flight), then every other wave's
        if (!prewaited) dg_wait_rt(c2 + c3);
        prewaited = false;
        __builtin_amdgcn_s_barrier();
        // into the slot of stage gs - 1, now free: stage hh + 3 of this pass, or of the next
        int c = 0;
        if (hh + 3 < S) c = issue(cur, ca, cn, hh + 3, gs + 3);
        else if (has_next) c = issue(nx, na_off, nn, hh + 3 - S, gs + 3);
        c2 = c3;
        c3 = c;
        if constexpr (NA > 0) {
          const uint8_t* sl = dRing + (gs % kDgSlots) * kDgSlotBytes;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(sl + boffs[s][0]);
            const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(sl + boffs[s][1]);
#pragma unroll
            for (int a = 0; a < NA; ++a) {
              const bf16x8 av = *reinterpret_cast<const bf16x8*>(sl + aoffs[s] + (2 * a + wm) * 2048);
              R[a][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b0, R[a][0], 0, 0, 0);
              R[a][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b1, R[a][1], 0, 0, 0);
            }
          }
        }
      }
      // wait now for the next pass's first stage: the stores below also count in
      // vmcnt and may complete in any order relative to the copies
      if (has_next) {
        dg_wait_rt(c2 + c3);
        prewaited = true;
      }
      if constexpr (NA > 0) {
        // a uniform base and 32-bit lane offsets, made opaque per tile so the
        // compiler does not hoist every store address of the pass at once
        float* yb = y + (size_t)(cur.r0 + cur.mb) * H + (size_t)cur.nt * kDgCols + 64 * wn;
#pragma unroll
        for (int a = 0; a < NA; ++a) {
          uint32_t o = (uint32_t)((32 * (2 * a + wm) + 4 * half) * H + col);
          asm volatile("" : "+v"(o));
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int dr = 8 * (j / 4) + (j % 4);
              if (32 * (2 * a + wm) + 4 * half + dr < cur.rows) yb[o + (uint32_t)(dr * H + 32 * c)] = R[a][c][j];
            }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    switch (na) {
      case 0: run(std::integral_constant<int, 0>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      default: run(std::integral_constant<int, 4>{}); break;
    }
    if (!has_next) break;
    cur = nx;
    ca[0] = na_off[0];
    ca[1] = na_off[1];
    cn = nn;
    item = item_n;
    g0 += S;
  }
}

// out[t, h .. h + 3] = sum_j w[t, j] * y[pos[t k + j], h .. h + 3], slot order
__global__ void k_down_combine(const float* __restrict__ y, int H, int k, const float* __restrict__ tw,
                               const int32_t* __restrict__ pos, float* __restrict__ out) {
  const int t = blockIdx.y;
  const int h = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
  if (h >= H) return;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const float wj = tw[t * k + j];
    const f32x4 v = *reinterpret_cast<const f32x4*>(y + (size_t)pos[t * k + j] * H + h);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = fmaf(wj, v[i], o[i]);
  }
  *reinterpret_cast<f32x4*>(out + (size_t)t * H + h) = o;
}

}  // namespace

template <typename AT>
static hipError_t down_gemv(const AT* act, int T, int I, const uint16_t* w, int H, int k, const int32_t* ids,
                            const float* tw, const int32_t* pos, float* out, hipStream_t st) {
  const dim3 grid(H / kDvRows, T);
  const int nq = cdiv(I, 256);
  switch (nq) {
    case 1: k_down_gemv_combine<1><<<grid, kDvThreads, 0, st>>>(act, I, w, H, k, ids, tw, pos, out); break;
    case 2: k_down_gemv_combine<2><<<grid, kDvThreads, 0, st>>>(act, I, w, H, k, ids, tw, pos, out); break;
    case 3: k_down_gemv_combine<3><<<grid, kDvThreads, 0, st>>>(act, I, w, H, k, ids, tw, pos, out); break;
    case 4: k_down_gemv_combine<4><<<grid, kDvThreads, 0, st>>>(act, I, w, H, k, ids, tw, pos, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_down_gemv_combine(const void* act, bool act_bf16, int T, int I, const uint16_t* w, int H, int k,
                                    const int32_t* ids, const float* tw, const int32_t* pos, float* out,
                                    hipStream_t st) {
  if (act_bf16) return down_gemv(static_cast<const uint16_t*>(act), T, I, w, H, k, ids, tw, pos, out, st);
  return down_gemv(static_cast<const float*>(act), T, I, w, H, k, ids, tw, pos, out, st);
}

hipError_t launch_down_gemm_combine(const void* act, bool act_bf16, int T, int I, const uint16_t* w, int E, int H,
                                    int k, const float* tw, const int32_t* expert_off, const int32_t* pos,
                                    uint16_t* a16, float* y, float* out, hipStream_t st) {
  hipError_t err;
  const uint16_t* a = static_cast<const uint16_t*>(act);
  if (!act_bf16) {
    const int64_t n8 = (int64_t)T * k * I / 8;
    k_f32_to_bf16<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(static_cast<const float*>(act), a16, n8);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    a = a16;
  }
  const int ntiles = H / kDgCols;
  const int grid = min(cdiv(E, kDgXcds) * kDgXcds * ntiles, kDgBlocks);   // both multiples of 8
  k_down_gemm<<<grid, kDgThreads, 0, st>>>(a, I, w, E, H, expert_off, y, ntiles);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  k_down_combine<<<dim3(cdiv(H / 4, 256), T), 256, 0, st>>>(y, H, k, tw, pos, out);
  return hipGetLastError();
}

}  // namespace i8h
