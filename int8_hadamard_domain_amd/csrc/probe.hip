// HBM read-bandwidth probe: the plainest kernel that reads a buffer once,
// the ceiling the HBM-bound kernels of the library are measured against on
// the same GPU. Not part of the product path (a separate library).
//
// Each lane reads 16-byte pieces with non-temporal loads, eight in flight
// (issued together, then folded), in a grid-stride pattern, so consecutive
// lanes read consecutive pieces and every wave load is 1 KB of one line run.
// The pieces are XOR-folded into one word per lane; the word is stored only
// if it equals a key the host passes (the host passes one no fold yields in
// practice), so the loads cannot be removed and nothing is written.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/i8h_probe.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ void __launch_bounds__(kThreads)
k_read_probe(const u32x4* __restrict__ p, uint64_t n16, uint32_t key, uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == key) sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" int i8h_read_probe(const void* buf, size_t bytes, int blocks, uint32_t key, uint32_t* sink,
                              void* stream) {
  if (!buf || !sink || bytes == 0 || (bytes % 16) != 0 || blocks <= 0) return -1;
  if ((reinterpret_cast<uintptr_t>(buf) % 16) != 0 || (reinterpret_cast<uintptr_t>(sink) % 4) != 0) return -1;
  k_read_probe<<<blocks, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(buf), (uint64_t)(bytes / 16), key, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
