// Router permutation: top-k over logits, per-expert histogram, exclusive scan
// and a stable scatter of (token, slot) pairs into expert-sorted order.
//
// Rule (the int8 card's model table, row "Weights", describes routed experts
// picked by a router and prints no rule): token t takes the k experts of
// largest logit, ties to the lower expert index; the weights are the softmax
// over the k chosen logits. Pairs p = t*k + j are grouped by expert with
// increasing p inside each expert (stable), which makes every integer
// output unique and lets the GPU reproduce it bit for bit: ranks come from
// ballots in lane order and fixed block order, never from atomic arrival order.
//
// Kernels
//   k_route_rows     per chunk of tokens (at most 256 pairs): top-k of every
//                    token (a wave per token) and the chunk's histogram over
//                    experts (LDS); optionally, in further workgroups of the
//                    same launch, the 128-wide Hadamard rotation of the token
//                    rows (the routing is the producer of the experts' input)
//   k_route_scatter  per chunk: totals + exclusive scan + in-chunk stable ranks
//   k_route_small    T <= 4: the three steps in one block (decode shape)

#include <mutex>

#include "common.hpp"
#include "launch.hpp"
#include "rotate.hpp"
#include "topk.hpp"

namespace i8h {

constexpr int kChunkPairs = 256;   // most pairs per histogram/scatter chunk
constexpr int kRouteThreads = 256;
constexpr int kRowThreads = 1024;  // k_route_rows: 16 waves, a token each at a time
constexpr int kRowWaves = kRowThreads / kWave;

// Chunks of whole tokens (a token's pairs never straddle two chunks), at
// most 256 pairs each, and small enough to give about 32 chunks when there
// are few tokens (each chunk is a workgroup of the routing kernel).
__host__ __device__ inline int chunk_tokens(int T, int k) {
  const int most = k >= kChunkPairs ? 1 : kChunkPairs / k;
  const int spread = (T + 31) / 32;
  return max(1, min(most, spread));
}

int64_t route_chunks(int T, int k) {
  const int tpc = chunk_tokens(T, k);
  return ((int64_t)T + tpc - 1) / tpc;
}

// --- top-k and chunk histogram; (ROT) rotation of the rows in the same launch
// Workgroups below nchunks route a chunk (a wave per token); with ROT the
// workgroups after them rotate the token rows, 16 lanes per 128-block, with
// the parallelism of a rotation kernel of their own (the rows do not depend
// on the routing), so the step saves a launch without rotating on fewer CUs.
template <int VPL, bool ROT>
__global__ void __launch_bounds__(kRowThreads)
k_route_rows(const float* __restrict__ logits, int T, int E, int k, int tpc, int nchunks,
             int32_t* __restrict__ ids, float* __restrict__ w, int32_t* __restrict__ hist,
             const uint16_t* x, uint16_t* xr, int K) {   // x and xr may be one buffer: not restrict
  if constexpr (ROT) {
    if ((int)blockIdx.x >= nchunks) {
      // x may be xr: each block is read whole by its 16 lanes before they write it
      const int KB = K / kGroup, j = threadIdx.x % 16;
      const int64_t b = (int64_t)(blockIdx.x - nchunks) * (blockDim.x / 16) + threadIdx.x / 16;
      const bool live = b < (int64_t)T * KB;
      const int64_t t = live ? b / KB : 0;
      const int kb = live ? (int)(b % KB) : 0;
      u32x4 xw = {0u, 0u, 0u, 0u};
      if (live) xw = *reinterpret_cast<const u32x4*>(x + t * K + kb * kGroup + 8 * j);
      const u32x4 o = fwht128_block(xw, j);   // every lane of the 16-lane row takes part
      if (live) *reinterpret_cast<u32x4*>(xr + t * K + kb * kGroup + 8 * j) = o;
      return;
    }
  }
  __shared__ int cnt[kMaxExperts];
  __shared__ uint64_t s_rank[kRowWaves][2 * kWave];   // the threshold top-k's scratch, a wave's own
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * tpc, t1 = min(T, t0 + tpc);
  for (int t = t0 + wave; t < t1; t += nwaves) {
    float v[VPL];
    load_logits<VPL>(logits + (size_t)t * E, E, lane, v);
    int id;
    float wt;
    // the threshold top-k packs the expert index in a byte (E <= 256)
    if constexpr (VPL <= 4) wave_topk_fast<VPL>(v, E, k, lane, id, wt, s_rank[wave]);
    else wave_topk<VPL>(v, E, k, lane, id, wt);
    if (lane < k) {
      ids[(size_t)t * k + lane] = id;
      w[(size_t)t * k + lane] = wt;
      atomicAdd(&cnt[id], 1);   // counts only: order does not matter
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Exclusive scan of tot[0..E) in LDS into off[0..E), block of 256 threads,
// each owning 4 consecutive experts. Returns nothing; off[E] is not written.
__device__ __forceinline__ void block_exclusive_scan(const int* tot, int* off, int E, int* wave_tot) {
  int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int base = tid * 4;
  int a[4];
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = (base + i < E) ? tot[base + i] : 0;
    s += a[i];
  }
  // inclusive wave scan of per-thread sums
  int inc = s;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) wave_tot[wave] = inc;
  __syncthreads();
  int wofs = 0;
  for (int w = 0; w < wave; ++w) wofs += wave_tot[w];
  int run = wofs + inc - s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (base + i < E) off[base + i] = run;
    run += a[i];
  }
}

// Stable in-block ranks: thread tid holds pair p (valid) with expert e.
// Returns the rank of p among the block's pairs of the same expert with a
// lower thread index. wcount is [4][E] in LDS, zero on entry, zero on exit.
__device__ __forceinline__ int block_stable_rank(bool valid, int e, int E, int nbits, int* wcount) {
  int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  uint64_t mask = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    bool bit = valid && ((e >> b) & 1);
    uint64_t bal = __ballot(bit);
    mask &= bit ? bal : ~bal;
  }
  uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int rank_w = __popcll(mask & lower);
  int cnt_w = __popcll(mask);
  if (valid && rank_w == 0) wcount[wave * E + e] = cnt_w;
  __syncthreads();
  int prefix = 0;
  if (valid)
    for (int w = 0; w < wave; ++w) prefix += wcount[w * E + e];
  __syncthreads();
  if (valid && rank_w == 0) wcount[wave * E + e] = 0;
  return prefix + rank_w;
}


// --- totals, scan and stable scatter of one chunk ------------------------
__global__ void __launch_bounds__(kRouteThreads)
k_route_scatter(const int32_t* __restrict__ ids, int P, int E, int nchunks, int cp,
                const int32_t* __restrict__ hist, int32_t* __restrict__ expert_off,
                int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos) {
  __shared__ int tot[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int pre[kMaxExperts];
  __shared__ int wcount[4 * kMaxExperts];
  __shared__ int wave_tot[4];
  int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    tot[e] = 0;
    pre[e] = 0;
  }
  for (int i = threadIdx.x; i < 4 * E; i += blockDim.x) wcount[i] = 0;
  __syncthreads();
  // tot[e] = sum of hist[cc][e] over all chunks, pre[e] = over chunks before
  // this one. The block reads the nchunks x E counts together, 16 independent
  // loads a thread at a time (one chain of loads per expert would cost a
  // round trip per chunk), and adds them with LDS atomics: integer sums, the
  // same in any order.
  const int n = nchunks * E;                          // < 2^31 (the caller checks)
  const int dcc = kRouteThreads / E, de = kRouteThreads % E;   // (cc, e) step of i += kRouteThreads
  for (int i0 = threadIdx.x; i0 < n; i0 += 16 * kRouteThreads) {
    int h[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + u * kRouteThreads;
      h[u] = i < n ? hist[i] : 0;
    }
    int cc = i0 / E, e = i0 - cc * E;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (h[u] != 0) {
        atomicAdd(&tot[e], h[u]);
        if (cc < c) atomicAdd(&pre[e], h[u]);
      }
      e += de;
      cc += dcc;
      if (e >= E) {  // de < E or de == kRouteThreads < E: one wrap at most
        e -= E;
        ++cc;
      }
    }
  }
  __syncthreads();
  block_exclusive_scan(tot, base, E, wave_tot);
  __syncthreads();
  if (c == 0) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) expert_off[e] = base[e];
    if (threadIdx.x == 0) expert_off[E] = P;
  }
  int p = c * cp + threadIdx.x;          // the chunk's pairs: cp <= 256 of them
  bool valid = (int)threadIdx.x < cp && p < P;
  int e = valid ? ids[p] : 0;
  int rank = block_stable_rank(valid, e, E, bits_for(E), wcount);
  if (valid) {
    int dst = base[e] + pre[e] + rank;
    sorted_pairs[dst] = p;
    pair_pos[p] = dst;
  }
}

// --- T <= 4: everything in one block --------------------------------------
template <int VPL>
__global__ void __launch_bounds__(kRouteThreads)
k_route_small(const float* __restrict__ logits, int T, int E, int k,
              int32_t* __restrict__ ids, float* __restrict__ w, int32_t* __restrict__ expert_off,
              int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos) {
  __shared__ int lds_ids[4 * kMaxTopk];
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int wcount[4 * kMaxExperts];
  __shared__ int wave_tot[4];
  int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  for (int i = threadIdx.x; i < 4 * E; i += blockDim.x) wcount[i] = 0;
  if (wave < T) {
    int id;
    float wt;
    float v[VPL];
    load_logits<VPL>(logits + (size_t)wave * E, E, lane, v);
    wave_topk<VPL>(v, E, k, lane, id, wt);
    if (lane < k) {
      ids[(size_t)wave * k + lane] = id;
      w[(size_t)wave * k + lane] = wt;
      lds_ids[wave * k + lane] = id;
    }
  }
  __syncthreads();
  int P = T * k;
  int p = threadIdx.x;
  bool valid = p < P;
  int e = valid ? lds_ids[p] : 0;
  if (valid) atomicAdd(&cnt[e], 1);
  __syncthreads();
  block_exclusive_scan(cnt, base, E, wave_tot);
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += blockDim.x) expert_off[i] = base[i];
  if (threadIdx.x == 0) expert_off[E] = P;
  int rank = block_stable_rank(valid, e, E, bits_for(E), wcount);
  if (valid) {
    int dst = base[e] + rank;
    sorted_pairs[dst] = p;
    pair_pos[p] = dst;
  }
}

size_t route_workspace_bytes(int T, int E, int k) {
  if (T <= 4) return 0;
  return (size_t)route_chunks(T, k) * (size_t)E * sizeof(int32_t);
}

// Scratch of the allocation-free routing call: the per-chunk histograms that
// the caller's workspace holds otherwise. Every GPU the library runs on keeps
// its own copy until the process ends. k_route_rows rewrites every histogram
// entry a call reads, so nothing needs clearing between calls.
static __device__ __align__(256) int32_t scratch[kRouteScratchBytes / sizeof(int32_t)];

hipError_t route_scratch(hipStream_t st, void** out) {
  // the array's name is a host-side stand-in: its device address comes from
  // hipGetSymbolAddress, once per device with that device current
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (st != nullptr) {
    int sdev = -1;
    e = hipStreamGetDevice(st, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != dev) return hipErrorInvalidDevice;   // the kernels would run on another GPU's copy
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

#define I8H_TOPK_DISPATCH(KERNEL, ...)                                   \
  do {                                                                   \
    if (vpl <= 1) KERNEL<1><<<grid, kRouteThreads, 0, st>>>(__VA_ARGS__);  \
    else if (vpl <= 2) KERNEL<2><<<grid, kRouteThreads, 0, st>>>(__VA_ARGS__); \
    else if (vpl <= 4) KERNEL<4><<<grid, kRouteThreads, 0, st>>>(__VA_ARGS__); \
    else if (vpl <= 8) KERNEL<8><<<grid, kRouteThreads, 0, st>>>(__VA_ARGS__); \
    else KERNEL<16><<<grid, kRouteThreads, 0, st>>>(__VA_ARGS__);        \
  } while (0)

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        int32_t* expert_off, int32_t* sorted_pairs, int32_t* pair_pos,
                        void* ws, const uint16_t* x, uint16_t* xr, int K, hipStream_t st) {
  int vpl = cdiv(E, kWave);
  if (T <= 4) {
    dim3 grid(1);
    I8H_TOPK_DISPATCH(k_route_small, logits, T, E, k, ids, w, expert_off, sorted_pairs, pair_pos);
    if (x != nullptr) return launch_fwht128(x, K, xr, K, T, K, st);
    return hipGetLastError();
  }
  const int tpc = chunk_tokens(T, k);
  const int64_t nchunks = route_chunks(T, k);
  const int threads = kWave * min(kRowWaves, tpc);   // a wave per token of the chunk, at most 16
  if (nchunks * E >= ((int64_t)1 << 31)) return hipErrorInvalidValue;  // histogram index range
  int32_t* hist = static_cast<int32_t*>(ws);
  const int P = T * k;
  const int nc = (int)nchunks;
  // rotation workgroups after the routing chunks: a 128-block per 16 lanes
  const int64_t rot_wgs = x != nullptr ? ((int64_t)T * (K / kGroup) + threads / 16 - 1) / (threads / 16) : 0;
  if (nc + rot_wgs >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int grid = nc + (int)rot_wgs;
#define I8H_ROWS(V)                                                                                      \
  do {                                                                                                   \
    if (x != nullptr)                                                                                    \
      k_route_rows<V, true><<<grid, threads, 0, st>>>(logits, T, E, k, tpc, nc, ids, w, hist, x, xr, K); \
    else                                                                                                 \
      k_route_rows<V, false><<<nc, threads, 0, st>>>(logits, T, E, k, tpc, nc, ids, w, hist, x, xr, K);  \
  } while (0)
  if (vpl <= 1) I8H_ROWS(1);
  else if (vpl <= 2) I8H_ROWS(2);
  else if (vpl <= 4) I8H_ROWS(4);
  else if (vpl <= 8) I8H_ROWS(8);
  else I8H_ROWS(16);
#undef I8H_ROWS
  k_route_scatter<<<nc, kRouteThreads, 0, st>>>(ids, P, E, nc, tpc * k, hist, expert_off, sorted_pairs, pair_pos);
  return hipGetLastError();
}

}  // namespace i8h
