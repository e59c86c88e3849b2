// Decode-shaped grouped int8 Hadamard-domain gate_up (few tokens per expert).
//
// Format (int8 card, model table row "Weights"): int8 codes -127..127 in the
// 128-wide Hadamard domain, one bf16 scale per row and 128 of K. For sorted
// row r of expert e and token t:
//   gu[r, n] = sum_g s[e, n, g] * sum_{kk in g} q[e, n, kk] * x_rot[t, kk]
//   act[r, i] = gelu_tanh(gu[r, i]) * gu[r, I + i]
// (act stored as float32, or by the grouped GEMV with AT = uint16_t as bf16
// rounded to nearest even from the float32 value)
//
// Work split: grid y = slot of a non-empty expert, grid x = groups of row
// pairs (i, I + i). Each wave owns RPW row pairs and issues all of their code
// loads at once (lane l reads the 16-byte pieces kk = 16 (l + 64 c) of every
// row: each wave load is 1 KB of one row), so many kilobytes are in flight per
// wave. Codes become float exactly (sign-extended byte converts), products
// with the bf16 activations are exact in float32 FMAs, each 16-value partial
// is scaled by its group's bf16 scale, and one transposing reduction (xor 32,
// 16, 8 keep half of the values each step; then xor 4, 2, 1) finishes all
// 2*RPW dot products of the wave in a fixed order. The codes are read once and
// reused for every token routed to the expert.
//
// Latency: at decode the whole kernel is one trip to HBM, so nothing that
// decides which codes to read may cost a trip of its own. The expert of a
// slot comes from one batch of expert_off loads (all issued before any is
// used) and ballots; the token of a row from a scalar load that overlaps the
// code stream.
//
// ROT = true takes unrotated activations and applies the 128-wide Hadamard
// rotation in the prologue: the 8 lanes holding one 128-block run four
// butterfly stages in registers and three across lanes (xor 1, 2, 4), scale
// by 1/sqrt(128) and round to bf16, exactly the activation the separate
// rotation call would produce up to float32 rounding order.
//
// k_route_gateup_decode adds the router in front (few tokens, at most 64
// pairs): every block ranks the logits of all tokens itself (a wave per
// token), groups the pairs by expert with ballots, picks the expert of its
// slot and goes on as above; block (0, 0) also stores the routing outputs.
// One launch then covers route -> rotate -> gate_up, and no block waits for
// another kernel's results. The four waves of a block split the rotation of a
// token row and share it through LDS; with a single token the row is fetched
// before the routing, and the rotation runs after the code loads are issued.

#include "common.hpp"
#include "launch.hpp"
#include "topk.hpp"
#include "xlane.hpp"

namespace i8h {

constexpr int kGemvThreads = 128;  // two waves: the decode grid spreads evenly over the CUs
constexpr int kGemvWaves = kGemvThreads / kWave;
// The routed decode kernel: every workgroup repeats the routing and the
// rotation of the token row, so four waves share them (half of that work
// per streamed byte against two-wave workgroups). A workgroup covers
// kDecWaves * RPW row pairs, which divides I (N % 64 == 0), so all of its
// waves have rows or none has.
constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kScanChunks = 4;  // expert_off entries per lane and round trip (E <= 256 in one)

// Expert owning the s-th non-empty run of expert_off (in expert order), with
// its first and one-past-last sorted row, or false. Same answer in every lane.
__device__ __forceinline__ bool nth_nonempty_expert(const int32_t* __restrict__ off, int E, int s, int lane,
                                                    int& e, int& r0, int& r1) {
  int seen = 0;
  for (int base = 0; base < E; base += kScanChunks * kWave) {
    int a[kScanChunks], b[kScanChunks];
#pragma unroll
    for (int c = 0; c < kScanChunks; ++c) {
      const int x = base + kWave * c + lane;
      a[c] = x < E ? off[x] : 0;
      b[c] = x < E ? off[x + 1] : 0;
    }
#pragma unroll
    for (int c = 0; c < kScanChunks; ++c) {
      uint64_t m = __ballot(b[c] > a[c]);
      const int cnt = __popcll(m);
      if (s < seen + cnt) {
        for (int i = seen; i < s; ++i) m &= m - 1;   // drop the lower set bits
        const int l = __ffsll((unsigned long long)m) - 1;
        e = base + kWave * c + l;
        r0 = __builtin_amdgcn_readlane(a[c], l);
        r1 = __builtin_amdgcn_readlane(b[c], l);
        return true;
      }
      seen += cnt;
    }
  }
  return false;
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

// Codes and scales of one wave's RPW row pairs, held in registers. A scale
// is kept as the aligned 4-byte word holding its bf16 bits and converted
// where it is used: converting it where it is loaded would make the wave wait
// for the load before it can do anything else.
template <int NCH, int RPW>
struct WaveRows {
  u32x4 cg[RPW][NCH], cu[RPW][NCH];
  uint32_t sg[RPW][NCH], su[RPW][NCH];
};

// The bf16 scale held in the high half of word w when odd, else in the low half.
__device__ __forceinline__ float scale_of_word(uint32_t w, int odd) {
  return __uint_as_float(odd ? (w & 0xffff0000u) : (w << 16));
}

// One token row as the lane reads it: the 16 values kk = 16 (lane + 64 c) ..
template <int NCH>
struct XRow {
  u32x4 a[NCH], b[NCH];
};

// A wave-uniform 64-bit value, held in scalar registers.
__device__ __forceinline__ size_t uniform_size(size_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((size_t)hi << 32) | lo;
}

template <int NCH, int RPW>
__device__ __forceinline__ void load_rows(WaveRows<NCH, RPW>& R, const int8_t* __restrict__ codes,
                                          const uint16_t* __restrict__ scales, int e, int N, int K, int i0,
                                          int lane) {
  // row bases are wave-uniform (scalar registers); a lane adds a 32-bit
  // offset, so every load takes the scalar-base form
  const int I = N / 2, G = K / kGroup;
  const uint32_t* sw = reinterpret_cast<const uint32_t*>(scales);  // 4-byte aligned
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const size_t rg = ((size_t)e * N + i0 + j) * G;  // element index of the row's first scale
    const size_t ru = rg + (size_t)I * G;
    const uint32_t* swg = sw + (rg >> 1);
    const uint32_t* swu = sw + (ru >> 1);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint32_t g = (uint32_t)min(16 * (lane + kWave * c), K - 16) / kGroup;
      R.sg[j][c] = swg[(((uint32_t)rg & 1u) + g) >> 1];
      R.su[j][c] = swu[(((uint32_t)ru & 1u) + g) >> 1];
    }
  }
  // in the order the dot products consume them (piece-major): loads complete
  // in issue order, so the first pieces can be used while the rest arrive
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint32_t kk = (uint32_t)min(16 * (lane + kWave * c), K - 16);  // pieces past K re-read the last one
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int8_t* rowg = codes + uniform_size(((size_t)e * N + i0 + j) * K);
      const int8_t* rowu = codes + uniform_size(((size_t)e * N + I + i0 + j) * K);
      R.cg[j][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowg + kk));
      R.cu[j][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowu + kk));
    }
  }
}

template <int NCH>
__device__ __forceinline__ void load_x(XRow<NCH>& X, const uint16_t* __restrict__ xr, int K, int lane) {
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int kk = min(16 * (lane + kWave * c), K - 16);
    X.a[c] = *reinterpret_cast<const u32x4*>(xr + kk);
    X.b[c] = *reinterpret_cast<const u32x4*>(xr + kk + 8);
  }
}

// The lane's activation values as float: bf16 -> float, rotated first when
// ROT (the 8 lanes of a 128-block together).
template <int NCH, bool ROT>
__device__ __forceinline__ void prep_x(const XRow<NCH>& X, float (&xv)[NCH][16], int lane) {
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      xv[c][2 * w] = bf16_lo(X.a[c][w]);
      xv[c][2 * w + 1] = bf16_hi(X.a[c][w]);
      xv[c][8 + 2 * w] = bf16_lo(X.b[c][w]);
      xv[c][8 + 2 * w + 1] = bf16_hi(X.b[c][w]);
    }
    if constexpr (ROT) rotate16(xv[c], lane);
  }
}

// gate_up (and act) of the wave's RPW row pairs for one token (its prepared
// activation values xv), stored at sorted row r. PIN_SCALES keeps the scale
// conversions inside the caller's row loop (where the activation row is
// prepared before the codes arrive, they must not wait for the scale loads).
template <int NCH, int RPW, bool PIN_SCALES, typename AT>
__device__ __forceinline__ void gemv_row(const WaveRows<NCH, RPW>& R, const float (&xv)[NCH][16], int K, int N,
                                         int i0, size_t r, float* __restrict__ gu, AT* __restrict__ act,
                                         int lane) {
  const int I = N / 2, G = K / kGroup;
  float v[2 * RPW];
#pragma unroll
  for (int q = 0; q < 2 * RPW; ++q) v[q] = 0.0f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    // a piece past K (a copy of the last one: finite) counts with weight 0
    const bool inside = 16 * (lane + kWave * c) < K;
    const int g = min(16 * (lane + kWave * c), K - 16) / kGroup;
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      // the codes (and with PIN_SCALES the scales) are loop-invariant over
      // rows; an empty asm keeps their conversion here (hoisted, it would hold
      // every code as a float)
      u32x4 qg = R.cg[j][c], qu = R.cu[j][c];
      uint32_t sg = R.sg[j][c], su = R.su[j][c];
      asm volatile("" : "+v"(qg), "+v"(qu));
      if constexpr (PIN_SCALES) asm volatile("" : "+v"(sg), "+v"(su));
      float pg0 = 0.0f, pg1 = 0.0f, pu0 = 0.0f, pu1 = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pg0 = fmaf(sbyte<0>(qg[w]), xv[c][4 * w + 0], pg0);
        pg1 = fmaf(sbyte<1>(qg[w]), xv[c][4 * w + 1], pg1);
        pg0 = fmaf(sbyte<2>(qg[w]), xv[c][4 * w + 2], pg0);
        pg1 = fmaf(sbyte<3>(qg[w]), xv[c][4 * w + 3], pg1);
        pu0 = fmaf(sbyte<0>(qu[w]), xv[c][4 * w + 0], pu0);
        pu1 = fmaf(sbyte<1>(qu[w]), xv[c][4 * w + 1], pu1);
        pu0 = fmaf(sbyte<2>(qu[w]), xv[c][4 * w + 2], pu0);
        pu1 = fmaf(sbyte<3>(qu[w]), xv[c][4 * w + 3], pu1);
      }
      // the element index (e N + i0 + j) G + g of the gate scale and the one
      // of the up scale (I rows later) have the parity of (i0 + j) G + g: N
      // and I are even
      const int odd = (((i0 + j) & G) ^ g) & 1;
      v[2 * j] = fmaf(inside ? scale_of_word(sg, odd) : 0.0f, pg0 + pg1, v[2 * j]);
      v[2 * j + 1] = fmaf(inside ? scale_of_word(su, odd) : 0.0f, pu0 + pu1, v[2 * j + 1]);
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
      gu[r * N + i0 + j] = g;
      gu[r * N + I + i0 + j] = u;
    }
    if (act) put_act(act, r * I + i0 + j, gelu_tanh(g) * u);
  }
}

template <int NCH, int RPW, bool ROT, typename AT>
__global__ void __launch_bounds__(kGemvThreads)
k_gateup_i8h_gemv(const uint16_t* __restrict__ xin, int K, const int8_t* __restrict__ codes,
                  const uint16_t* __restrict__ scales, int E, int N, int k,
                  const int32_t* __restrict__ expert_off, const int32_t* __restrict__ sorted_pairs,
                  float* __restrict__ gu, AT* __restrict__ act) {
  static_assert(RPW == 2 || RPW == 4, "2*RPW values per lane are folded over bits 5..");
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: row bases in SGPRs
  const int I = N / 2;
  const int i0 = (blockIdx.x * kGemvWaves + wave) * RPW;  // I % RPW == 0, so all RPW rows exist
  if (i0 >= I) return;
  int e, r0, r1;
  if (!nth_nonempty_expert(expert_off, E, blockIdx.y, lane, e, r0, r1)) return;
  // issue order: the first row's token (scalar load), scales and codes, then
  // that row's activations; the next row's activations are fetched while the
  // current row is being reduced
  const int p0 = sorted_pairs[r0];
  __builtin_amdgcn_sched_barrier(0);  // (the scheduler would otherwise wait for p0 before the code loads)
  WaveRows<NCH, RPW> R;
  load_rows(R, codes, scales, e, N, K, i0, lane);
  __builtin_amdgcn_sched_barrier(0);
  int t = p0 / k;
  XRow<NCH> X;
  load_x(X, xin + (size_t)t * K, K, lane);
  for (int r = r0; r < r1; ++r) {
    float xv[NCH][16];
    prep_x<NCH, ROT>(X, xv, lane);
    if (r + 1 < r1) {
      t = sorted_pairs[r + 1] / k;
      load_x(X, xin + (size_t)t * K, K, lane);
    }
    gemv_row<NCH, RPW, false>(R, xv, K, N, i0, (size_t)r, gu, act, lane);
  }
}

// The rotation of one token row is shared by the waves of a workgroup: wave
// w rotates the pieces c = w, w + kDecWaves, .. (64 lanes x 16 values each)
// and leaves them as bf16 in LDS, where every wave reads the whole row.
template <int NCH>
struct RotShare {
  static constexpr int kN = (NCH + kDecWaves - 1) / kDecWaves;
  XRow<kN> X;

  __device__ __forceinline__ void load(const uint16_t* __restrict__ xr, int K, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      if (wave + kDecWaves * i >= NCH) break;  // uniform in the wave
      const int kk = min(16 * (lane + kWave * (wave + kDecWaves * i)), K - 16);  // past K: a copy (weight 0 later)
      X.a[i] = *reinterpret_cast<const u32x4*>(xr + kk);
      X.b[i] = *reinterpret_cast<const u32x4*>(xr + kk + 8);
    }
  }

  __device__ __forceinline__ void rotate_to(uint16_t* s_xr, int wave, int lane) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int c = wave + kDecWaves * i;
      if (c >= NCH) break;  // uniform in the wave
      float xv[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        xv[2 * w] = bf16_lo(X.a[i][w]);
        xv[2 * w + 1] = bf16_hi(X.a[i][w]);
        xv[8 + 2 * w] = bf16_lo(X.b[i][w]);
        xv[8 + 2 * w + 1] = bf16_hi(X.b[i][w]);
      }
      rotate16(xv, lane);
      u32x4 lo, hi;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        lo[w] = pack_bf16x2(xv[2 * w], xv[2 * w + 1]);       // exact: already bf16 values
        hi[w] = pack_bf16x2(xv[8 + 2 * w], xv[8 + 2 * w + 1]);
      }
      u32x4* dst = reinterpret_cast<u32x4*>(s_xr + 16 * (lane + kWave * c));
      dst[0] = lo;
      dst[1] = hi;
    }
  }
};

template <int NCH>
__device__ __forceinline__ void read_rotated(const uint16_t* s_xr, float (&xv)[NCH][16], int lane) {
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const u32x4* src = reinterpret_cast<const u32x4*>(s_xr + 16 * (lane + kWave * c));
    const u32x4 a = src[0], b = src[1];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      xv[c][2 * w] = bf16_lo(a[w]);
      xv[c][2 * w + 1] = bf16_hi(a[w]);
      xv[c][8 + 2 * w] = bf16_lo(b[w]);
      xv[c][8 + 2 * w + 1] = bf16_hi(b[w]);
    }
  }
}

// One token: the k chosen experts hold one pair each, so the sorted row of a
// workgroup's slot s is s and its expert is the s-th chosen one in index
// order. Every wave finds the chosen set itself (topk_mask: registers and
// ballots only), picks its expert and issues its code loads, with no LDS
// round trip and no barrier before them. Workgroup (0, 0) then ranks the
// chosen experts (slot order, softmax weights) and stores the routing
// outputs while its codes arrive.
template <int NCH, int RPW, int VPL>
__device__ __forceinline__ void decode_one_token(const float* __restrict__ logits, const uint16_t* __restrict__ x,
                                                 int K, const int8_t* __restrict__ codes,
                                                 const uint16_t* __restrict__ scales, int E, int N, int k,
                                                 int32_t* __restrict__ ids_out, float* __restrict__ w_out,
                                                 int32_t* __restrict__ expert_off,
                                                 int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos,
                                                 float* __restrict__ gu, float* __restrict__ act,
                                                 uint64_t* s_rank, uint16_t* s_xr, int wave, int lane) {
  const int I = N / 2;
  const bool writer = blockIdx.x == 0 && blockIdx.y == 0;
  float lv[VPL];
  load_logits<VPL>(logits, E, lane, lv);
  RotShare<NCH> share;
  share.load(x, K, wave, lane);                 // needed whatever the routing
  uint64_t chosen[VPL];
  topk_mask<VPL>(lv, E, k, lane, chosen);
  // the expert of this block's slot: the blockIdx.y-th chosen one in index order
  int e = -1, rem = blockIdx.y;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = __popcll(chosen[i]);
    if (e < 0) {
      if (rem < c) {
        uint64_t m = chosen[i];
        for (int q = 0; q < rem; ++q) m &= m - 1;
        e = kWave * i + __ffsll((unsigned long long)m) - 1;
      } else {
        rem -= c;
      }
    }
  }
  // routing outputs from the chosen set (ranks and weights from the ranked
  // top-k of the same rule): ids and weights in slot order, the sorted row of
  // pair j = the number of chosen experts below its expert, expert_off
  auto store_routing = [&]() {
    if (wave != 0) return;
    int id;
    float wt;
    wave_topk_fast<VPL>(lv, E, k, lane, id, wt, s_rank);
    auto chosen_below = [&](int ex) {
      int c = 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int lo = ex - kWave * i;           // chosen entries of word i with index < ex
        c += lo <= 0 ? 0 : lo >= kWave ? __popcll(chosen[i]) : __popcll(chosen[i] & ((1ull << lo) - 1));
      }
      return c;
    };
    if (lane < k) {
      const int row = chosen_below(id);
      ids_out[lane] = id;
      w_out[lane] = wt;
      sorted_pairs[row] = lane;
      pair_pos[lane] = row;
    }
    for (int ex = lane; ex <= E; ex += kWave) expert_off[ex] = chosen_below(ex);
  };
  const int i0 = (blockIdx.x * kDecWaves + wave) * RPW;
  if (e < 0 || i0 >= I) {                       // the same for every wave of the block
    if (writer) store_routing();
    return;
  }
  __builtin_amdgcn_sched_barrier(0);
  WaveRows<NCH, RPW> R;
  load_rows(R, codes, scales, e, N, K, i0, lane);
  __builtin_amdgcn_sched_barrier(0);
  if (writer) store_routing();
  share.rotate_to(s_xr, wave, lane);            // runs while the codes arrive
  __syncthreads();
  float xv[NCH][16];
  read_rotated<NCH>(s_xr, xv, lane);
  gemv_row<NCH, RPW, true>(R, xv, K, N, i0, (size_t)blockIdx.y, gu, act, lane);
}

template <int NCH, int RPW, int VPL>
__global__ void __launch_bounds__(kDecThreads)
k_route_gateup_decode(const float* __restrict__ logits, const uint16_t* __restrict__ x, int T, int K,
                      const int8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int E, int N, int k,
                      int32_t* __restrict__ ids_out, float* __restrict__ w_out, int32_t* __restrict__ expert_off,
                      int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos,
                      float* __restrict__ gu, float* __restrict__ act) {
  static_assert(32 % (kDecWaves * RPW) == 0, "a workgroup's row pairs divide I");
  __shared__ int s_ids[kWave];
  __shared__ uint64_t s_rank[kDecWaves][2 * kWave];                       // top-k scratch, a wave's own
  __shared__ __attribute__((aligned(16))) uint16_t s_xr[NCH * 16 * kWave];  // rotated row, bf16
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: row bases in SGPRs
  const int I = N / 2;
  const bool writer = blockIdx.x == 0 && blockIdx.y == 0;  // stores the routing outputs
  const int P = T * k;                                     // <= 64
  if (T == 1) {
    decode_one_token<NCH, RPW, VPL>(logits, x, K, codes, scales, E, N, k, ids_out, w_out, expert_off, sorted_pairs,
                                    pair_pos, gu, act, s_rank[0], s_xr, wave, lane);
    return;
  }

  // the first token's logits go out first; with a single token its
  // activations are needed whatever the routing, so they follow at once and
  // are in registers long before the code stream
  float lv[VPL];
  if (wave < T) load_logits<VPL>(logits + (size_t)wave * E, E, lane, lv);
  RotShare<NCH> share;
  if (T == 1) share.load(x, K, wave, lane);

  // top-k of every token, a wave per token
  for (int t = wave; t < T; t += kDecWaves) {
    int id;
    float wt;
    if (t != wave) load_logits<VPL>(logits + (size_t)t * E, E, lane, lv);
    wave_topk_fast<VPL>(lv, E, k, lane, id, wt, s_rank[wave]);
    if (lane < k) {
      s_ids[t * k + lane] = id;
      if (writer) {
        ids_out[t * k + lane] = id;
        w_out[t * k + lane] = wt;
      }
    }
  }
  __syncthreads();

  // group the pairs by expert (each wave on its own, same result everywhere):
  // below = the first sorted row of the pair's expert, rank = the pair's place
  // inside it, slot = the expert's place among the non-empty ones, same = the
  // lanes (pairs) of the expert
  const bool valid = lane < P;
  const int ep = valid ? s_ids[lane] : 0;
  int below, rank, slot;
  uint64_t same;
  if (T == 1) {
    // one token: its k experts are distinct and hold one pair each, so the
    // sorted row and the slot of pair p are the number of chosen experts below
    // its own (k LDS broadcast reads instead of a ballot per index bit)
    int c = 0;
    for (int q = 0; q < P; ++q) c += s_ids[q] < ep;
    below = c;
    rank = 0;
    slot = c;
    same = 1ull << lane;
  } else {
    const PairGroup pg = wave_group_by_expert(valid, ep, bits_for(E));
    below = __popcll(pg.lt);
    rank = __popcll(pg.eq & lanes_below(lane));
    const uint64_t first = __ballot(valid && rank == 0);   // one lane per non-empty expert
    slot = __popcll(pg.lt & first);
    same = pg.eq;
  }
  // the routing outputs: stored by block (0, 0) after its own code loads
  // are on their way (below), or here if it has no rows to work on
  auto store_routing = [&]() {
    if (wave == 0 && valid) {
      sorted_pairs[below + rank] = lane;
      pair_pos[lane] = below + rank;
    }
    // expert_off[e] = number of pairs routed to experts below e
    for (int e = threadIdx.x; e <= E; e += kDecThreads) {
      int c = 0;
      for (int q = 0; q < P; ++q) c += s_ids[q] < e;
      expert_off[e] = c;
    }
  };
  // all waves of a workgroup see the same slot and (kDecWaves * RPW divides
  // I) the same i0 range, so they leave together and meet at the barriers below
  const uint64_t mine = __ballot(valid && rank == 0 && slot == (int)blockIdx.y);
  const int i0 = (blockIdx.x * kDecWaves + wave) * RPW;
  if (mine == 0 || i0 >= I) {
    if (writer) store_routing();
    return;
  }
  const int L = __ffsll((unsigned long long)mine) - 1;
  const int e = __builtin_amdgcn_readlane(ep, L);
  const int r0 = __builtin_amdgcn_readlane(below, L);
  uint64_t rows = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(same >> 32), L) << 32) |
                  (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)same, L);

  int p = __ffsll((unsigned long long)rows) - 1;  // pairs of the expert in increasing order
  rows &= rows - 1;
  if (T != 1) share.load(x + (size_t)(p / k) * K, K, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  WaveRows<NCH, RPW> R;
  load_rows(R, codes, scales, e, N, K, i0, lane);
  __builtin_amdgcn_sched_barrier(0);
  if (writer) store_routing();
  for (int r = r0; p >= 0; ++r) {
    if (r != r0) __syncthreads();        // the previous row is read by every wave
    share.rotate_to(s_xr, wave, lane);   // runs while the codes arrive
    __syncthreads();
    float xv[NCH][16];
    read_rotated<NCH>(s_xr, xv, lane);
    __builtin_amdgcn_sched_barrier(0);
    p = rows ? __ffsll((unsigned long long)rows) - 1 : -1;
    rows &= rows - 1;
    if (p >= 0) share.load(x + (size_t)(p / k) * K, K, wave, lane);
    gemv_row<NCH, RPW, true>(R, xv, K, N, i0, (size_t)r, gu, act, lane);
  }
}

template <bool ROT, typename AT>
static hipError_t launch_gemv(const uint16_t* x, int T, int K, const int8_t* codes, const uint16_t* scales, int E,
                              int N, int k, const int32_t* expert_off, const int32_t* sorted_pairs, float* gu,
                              AT* act, hipStream_t st) {
  int P = T * k;
  int slots = P < E ? P : E;  // at most this many experts can be non-empty
  int I = N / 2;
  int nch = cdiv(K, 16 * kWave);
  if (nch <= 1) {
    dim3 grid(cdiv(I, kGemvWaves * 4), slots);
    k_gateup_i8h_gemv<1, 4, ROT><<<grid, kGemvThreads, 0, st>>>(x, K, codes, scales, E, N, k, expert_off,
                                                                sorted_pairs, gu, act);
  } else if (nch <= 2) {
    dim3 grid(cdiv(I, kGemvWaves * 2), slots);
    k_gateup_i8h_gemv<2, 2, ROT><<<grid, kGemvThreads, 0, st>>>(x, K, codes, scales, E, N, k, expert_off,
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
                                  const int32_t* sorted_pairs, float* gu, void* act, bool act_bf16,
                                  hipStream_t st) {
  if (act_bf16)
    return launch_gemv<false>(xrot, T, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu,
                              static_cast<uint16_t*>(act), st);
  return launch_gemv<false>(xrot, T, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu,
                            static_cast<float*>(act), st);
}

hipError_t launch_gateup_i8h_gemv_rot(const uint16_t* x, int T, int K, const int8_t* codes,
                                      const uint16_t* scales, int E, int N, int k, const int32_t* expert_off,
                                      const int32_t* sorted_pairs, float* gu, float* act, hipStream_t st) {
  return launch_gemv<true>(x, T, K, codes, scales, E, N, k, expert_off, sorted_pairs, gu, act, st);
}

template <int NCH, int RPW>
static void launch_decode(dim3 grid, int vpl, const float* logits, const uint16_t* x, int T, int K,
                          const int8_t* codes, const uint16_t* scales, int E, int N, int k, int32_t* ids, float* w,
                          int32_t* expert_off, int32_t* sorted_pairs, int32_t* pair_pos, float* gu, float* act,
                          hipStream_t st) {
#define I8H_DECODE_ARGS logits, x, T, K, codes, scales, E, N, k, ids, w, expert_off, sorted_pairs, pair_pos, gu, act
  if (vpl <= 1) k_route_gateup_decode<NCH, RPW, 1><<<grid, kDecThreads, 0, st>>>(I8H_DECODE_ARGS);
  else if (vpl <= 2) k_route_gateup_decode<NCH, RPW, 2><<<grid, kDecThreads, 0, st>>>(I8H_DECODE_ARGS);
  else k_route_gateup_decode<NCH, RPW, 4><<<grid, kDecThreads, 0, st>>>(I8H_DECODE_ARGS);
#undef I8H_DECODE_ARGS
}

hipError_t launch_route_gateup_decode(const float* logits, const uint16_t* x, int T, int K, const int8_t* codes,
                                      const uint16_t* scales, int E, int N, int k, int32_t* ids, float* w,
                                      int32_t* expert_off, int32_t* sorted_pairs, int32_t* pair_pos, float* gu,
                                      float* act, hipStream_t st) {
  int P = T * k;
  int slots = P < E ? P : E;
  int I = N / 2;
  int nch = cdiv(K, 16 * kWave);
  int vpl = cdiv(E, kWave);
  if (nch <= 1) {
    launch_decode<1, 4>(dim3(cdiv(I, kDecWaves * 4), slots), vpl, logits, x, T, K, codes, scales, E, N, k, ids, w,
                        expert_off, sorted_pairs, pair_pos, gu, act, st);
  } else if (nch <= 2) {
    launch_decode<2, 2>(dim3(cdiv(I, kDecWaves * 2), slots), vpl, logits, x, T, K, codes, scales, E, N, k, ids, w,
                        expert_off, sorted_pairs, pair_pos, gu, act, st);
  } else {
    launch_decode<4, 2>(dim3(cdiv(I, kDecWaves * 2), slots), vpl, logits, x, T, K, codes, scales, E, N, k, ids, w,
                        expert_off, sorted_pairs, pair_pos, gu, act, st);
  }
  return hipGetLastError();
}

}  // namespace i8h
