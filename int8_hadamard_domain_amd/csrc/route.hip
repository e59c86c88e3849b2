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
//   k_route_topk     one wave per token (grid T/4 x 256 threads)
//   k_route_count    per chunk of 256 pairs: histogram over experts (LDS)
//   k_route_scatter  per chunk: totals + exclusive scan + in-chunk stable ranks
//   k_route_small    T <= 4: the three steps in one block (decode shape)

#include <mutex>

#include "common.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace i8h {

constexpr int kChunkPairs = 256;   // pairs per histogram/scatter block
constexpr int kRouteThreads = 256;

template <int VPL>
__global__ void __launch_bounds__(kRouteThreads)
k_route_topk(const float* __restrict__ logits, int T, int E, int k,
             int32_t* __restrict__ ids, float* __restrict__ w) {
  int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  int t = blockIdx.x * (kRouteThreads / kWave) + wave;
  if (t >= T) return;
  int id;
  float wt;
  float v[VPL];
  load_logits<VPL>(logits + (size_t)t * E, E, lane, v);
  wave_topk<VPL>(v, E, k, lane, id, wt);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    w[(size_t)t * k + lane] = wt;
  }
}

// --- histogram of one chunk of pairs -------------------------------------
__global__ void __launch_bounds__(kRouteThreads)
k_route_count(const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ hist) {
  __shared__ int cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  int p = blockIdx.x * kChunkPairs + threadIdx.x;
  if (p < P) atomicAdd(&cnt[ids[p]], 1);   // counts only: order does not matter
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
k_route_scatter(const int32_t* __restrict__ ids, int P, int E, int nchunks,
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
  int p = c * kChunkPairs + threadIdx.x;
  bool valid = p < P;
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
  size_t P = (size_t)T * k;
  size_t nchunks = (P + kChunkPairs - 1) / kChunkPairs;
  return nchunks * (size_t)E * sizeof(int32_t);
}

// Scratch of the allocation-free routing call: the per-chunk histograms that
// the caller's workspace holds otherwise. Every GPU the library runs on keeps
// its own copy until the process ends. k_route_count rewrites every histogram
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
                        void* ws, hipStream_t st) {
  int vpl = cdiv(E, kWave);
  if (T <= 4) {
    dim3 grid(1);
    I8H_TOPK_DISPATCH(k_route_small, logits, T, E, k, ids, w, expert_off, sorted_pairs, pair_pos);
    return hipGetLastError();
  }
  {
    dim3 grid(cdiv(T, kRouteThreads / kWave));
    I8H_TOPK_DISPATCH(k_route_topk, logits, T, E, k, ids, w);
  }
  int P = T * k;
  int nchunks = cdiv(P, kChunkPairs);
  if ((int64_t)nchunks * E >= ((int64_t)1 << 31)) return hipErrorInvalidValue;  // histogram index range
  int32_t* hist = static_cast<int32_t*>(ws);
  k_route_count<<<nchunks, kRouteThreads, 0, st>>>(ids, P, E, hist);
  k_route_scatter<<<nchunks, kRouteThreads, 0, st>>>(ids, P, E, nchunks, hist, expert_off, sorted_pairs,
                                                     pair_pos);
  return hipGetLastError();
}

}  // namespace i8h
