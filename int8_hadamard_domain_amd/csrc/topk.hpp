// Wave-level routing pieces shared by the router kernels and the fused decode
// kernel.
//
// Rule (the int8 card's model table, row "Weights", describes routed experts
// picked by a router and prints no rule): token t takes the k experts of
// largest logit, ties to the lower expert index, weights = softmax over the k
// chosen logits. Pairs p = t*k + j are grouped by expert with increasing p
// inside each expert.
#pragma once

#include "common.hpp"
#include "xlane.hpp"

namespace i8h {

// Top-k of one token by one wave. Lane l holds logits e = l + 64 i. Each
// round takes the largest open order key (a wave maximum) and, among the open
// entries equal to it, the lowest expert index (ballots in index order), then
// retires that entry: the order "larger value first, then lower index", with
// NaN after every number. Lane j < k returns the j-th choice (always an
// index in [0, E)) and its softmax weight; other lanes return id -1.
template <int VPL>
__device__ __forceinline__ void load_logits(const float* __restrict__ row, int E, int lane, float (&v)[VPL]) {
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    v[i] = e < E ? row[e] : -INFINITY;
  }
}

// Order-preserving map of a float32 to an unsigned key (+0 and -0 map alike).
// Every NaN maps to 0, below the key of -inf (0x007fffff): a NaN logit ranks
// after every number, and NaNs among themselves by index like any tie. No
// real logit has key 0, so key_logit(0) gives a NaN back.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);    // -0 + 0 = +0
  const uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return v == v ? k : 0u;
}

// Inverse of order_key on the keys of numbers; key 0 (a NaN) gives a NaN.
__device__ __forceinline__ float key_logit(uint32_t key) {
  if (key == 0u) return __uint_as_float(0x7fc00000u);
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

template <int VPL>
__device__ __forceinline__ void wave_topk(const float (&v)[VPL], int E, int k, int lane, int& id, float& weight) {
  // ranks the order keys: integer maxima need no NaN handling, and a NaN
  // (key 0) still takes part, after every number. Entries past E are never
  // open, and k <= E, so every round finds an open entry.
  uint32_t kv[VPL];
  uint32_t open = 0;  // bit i: entry i of this lane not yet taken
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    kv[i] = order_key(v[i]);
    if (lane + kWave * i < E) open |= 1u << i;
  }
  int my_id = 0;
  uint32_t my_key = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if ((open >> i) & 1u) m = max(m, kv[i]);
    m = max(m, (uint32_t)xor_lane_i<1>((int)m));
    m = max(m, (uint32_t)xor_lane_i<2>((int)m));
    m = max(m, (uint32_t)xor_lane_i<4>((int)m));
    m = max(m, (uint32_t)xor_lane_i<8>((int)m));
    m = max(m, (uint32_t)xor_lane_i<16>((int)m));
    m = max(m, (uint32_t)xor_lane_i<32>((int)m));
    int best = -1;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const uint64_t b = __ballot(((open >> i) & 1u) && kv[i] == m);
      if (best < 0 && b != 0) best = kWave * i + __ffsll((unsigned long long)b) - 1;
    }
    if ((best % kWave) == lane) open &= ~(1u << (best / kWave));
    if (lane == j) {
      my_id = best;
      my_key = m;
    }
  }
  const float my_logit = key_logit(my_key);
  const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_logit), 0));
  float ex = lane < k ? expf(my_logit - l0) : 0.0f;
  float sum = wave_sum(ex);
  id = lane < k ? my_id : -1;
  weight = lane < k ? ex / sum : 0.0f;
}

// The same top-k, faster when the k largest stand out (the usual case for
// router logits). The 4 VPL maxima of 16-lane rows (8 maxima of 8-lane
// groups when VPL == 1) are values of distinct entries, so the smallest of
// them, tau, is at most the k-th largest when k does not exceed their number:
// the entries >= tau hold the whole answer, ties at the boundary included.
// They are written to `scratch` (a wave's own 128 x 8 bytes of LDS) as unique
// keys (order key << 8 | 255 - index: larger value first, then lower index),
// each ranked by counting the keys above it, and the first k are taken in
// rank order. More than 64 candidates, k above the number of groups, or a
// tau at or below the key of -inf (a row group of NaNs or -inf only) fall
// back to wave_topk. Same ids and weights as wave_topk.
template <int VPL>
__device__ __forceinline__ void wave_topk_fast(const float (&v)[VPL], int E, int k, int lane, int& id, float& weight,
                                               uint64_t* scratch) {
  constexpr int kGroups = VPL == 1 ? 8 : 4 * VPL;
  // the threshold on the order keys (unsigned, monotone in the logit):
  // integer max and min need no NaN handling between the cross-lane steps;
  // entries past E take key 0, below every logit's key
  uint32_t kv[VPL];
  uint32_t tau = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    kv[i] = lane + kWave * i < E ? order_key(v[i]) : 0u;
    uint32_t m = kv[i];
    m = max(m, (uint32_t)xor_lane_i<1>((int)m));
    m = max(m, (uint32_t)xor_lane_i<2>((int)m));
    m = max(m, (uint32_t)xor_lane_i<4>((int)m));
    if constexpr (VPL > 1) m = max(m, (uint32_t)xor_lane_i<8>((int)m));
    tau = min(tau, m);
  }
  if constexpr (VPL == 1) tau = min(tau, (uint32_t)xor_lane_i<8>((int)tau));
  tau = min(tau, (uint32_t)xor_lane_i<16>((int)tau));
  tau = min(tau, (uint32_t)xor_lane_i<32>((int)tau));
  uint64_t cm[VPL];
  int C = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    cm[i] = __ballot(kv[i] >= tau && lane + kWave * i < E);
    C += __popcll(cm[i]);
  }
  // a row group with no logit above -inf gives no usable threshold
  if (k > kGroups || C > kWave || tau <= order_key(-INFINITY)) {
    wave_topk<VPL>(v, E, k, lane, id, weight);
    return;
  }
  // candidates in index order, element i of lane l after every earlier one
  int base = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if ((cm[i] >> lane) & 1) {
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(cm[i] >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)cm[i], 0u));
      scratch[pos] = ((uint64_t)kv[i] << 8) | (uint64_t)(255 - (lane + kWave * i));
    }
    base += __popcll(cm[i]);
  }
  __builtin_amdgcn_wave_barrier();
  const uint64_t mine = lane < C ? scratch[lane] : 0ull;
  int r = 0;
  for (int j = 0; j < C; ++j) r += scratch[j] > mine ? 1 : 0;
  __builtin_amdgcn_wave_barrier();
  if (lane < C && r < k) scratch[kWave + r] = mine;
  __builtin_amdgcn_wave_barrier();
  int my_id = -1;
  float my_logit = 0.0f;
  if (lane < k) {
    const uint64_t t = scratch[kWave + lane];
    const uint32_t key = (uint32_t)(t >> 8);
    my_id = 255 - (int)(t & 0xffu);
    my_logit = key_logit(key);
  }
  const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_logit), 0));
  float ex = lane < k ? expf(my_logit - l0) : 0.0f;
  float sum = wave_sum(ex);
  id = my_id;
  weight = lane < k ? ex / sum : 0.0f;
}

// The set of the k largest entries of one token (the same rule: larger
// order key first, ties to the lower index, NaN last), as one bit per lane
// for each of a lane's VPL entries, with no LDS: bisection over the 32 bits
// of the order keys for the largest threshold with at least k keys at or
// above it (each step one ballot count per entry), then every key above the
// threshold and, of the keys equal to it, the lowest indices. The search
// stops early once exactly k keys lie at or above a candidate: those are the
// k largest, ties impossible. Wave-uniform result; k <= E.
template <int VPL>
__device__ __forceinline__ void topk_mask(const float (&v)[VPL], int E, int k, int lane, uint64_t (&chosen)[VPL]) {
  // entries past E take key 0 like NaN: no candidate (never 0) counts them,
  // and only a threshold of 0 needs the index bound (ties below)
  uint32_t kv[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) kv[i] = lane + kWave * i < E ? order_key(v[i]) : 0u;
  uint32_t thr = 0;
  bool exact = false;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = thr | (1u << b);
    int c = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) c += __popcll(__ballot(kv[i] >= cand));
    if (c >= k) {
      thr = cand;
      if (c == k) {
        exact = true;
        break;
      }
    }
  }
  int need = k;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    chosen[i] = __ballot(exact ? kv[i] >= thr : kv[i] > thr);   // thr > 0 when exact
    need -= __popcll(chosen[i]);
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    uint64_t eq = __ballot(kv[i] == thr && lane + kWave * i < E);
    while (need > 0 && eq != 0) {       // ties at the threshold: lowest indices first
      chosen[i] |= eq & (~eq + 1);
      eq &= eq - 1;
      --need;
    }
  }
}

// Grouping of up to 64 pairs by expert inside one wave: lane p holds pair p
// (valid) routed to expert e (0 <= e < 2^nbits). Radix over the bits of e,
// most significant first, with one ballot per bit:
//   lt = lanes whose expert is smaller than e, eq = lanes with expert e.
// Then |lt| is the expert's first sorted row and |eq below p| the pair's rank
// inside its expert (the stable order).
struct PairGroup {
  uint64_t lt, eq;
};
__device__ __forceinline__ PairGroup wave_group_by_expert(bool valid, int e, int nbits) {
  PairGroup g;
  g.lt = 0;
  g.eq = __ballot(valid);
  for (int b = nbits - 1; b >= 0; --b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t B = __ballot(bit);
    if (bit) {
      g.lt |= g.eq & ~B;
      g.eq &= B;
    } else {
      g.eq &= ~B;
    }
  }
  if (!valid) g.eq = 0;
  return g;
}

__device__ __forceinline__ uint64_t lanes_below(int lane) { return lane == 0 ? 0ull : (~0ull >> (kWave - lane)); }

__device__ __forceinline__ int bits_for(int E) {
  int nb = 0;
  while ((1 << nb) < E) ++nb;
  return nb;
}

}  // namespace i8h
