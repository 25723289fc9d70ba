// Streaming-read probe: the practical HBM read ceiling that the decode
// kernels are measured against (next to the vendor peak).
//
// Each block reads one contiguous chunk of the buffer with 16-byte
// nontemporal loads, four in flight per thread, and folds the words into an
// XOR so the loads are live; one word per block is written to `sink`.
#include "common.hpp"
#include "kernels.hpp"

namespace mikv {

namespace {

typedef unsigned probe_u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const probe_u32x4* __restrict__ p, int64_t n16,
                                                                     int64_t chunk, uint32_t* __restrict__ sink) {
  const int64_t begin = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t end = min(n16, begin + chunk);
  uint32_t x = 0;
  constexpr int64_t kStep = static_cast<int64_t>(kProbeThreads) * kProbeUnroll;
  for (int64_t i = begin + threadIdx.x; i < end; i += kStep) {
    probe_u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const int64_t j = i + static_cast<int64_t>(u) * kProbeThreads;
      v[u] = (j < end) ? __builtin_nontemporal_load(p + j) : probe_u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // one word per block: the XOR over the block's threads
  __shared__ uint32_t red[kProbeThreads];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int k = 0; k < kProbeThreads; ++k) t ^= red[k];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* p, size_t bytes, int blocks, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  const int64_t chunk = (n16 + blocks - 1) / blocks;
  read_probe_kernel<<<blocks, kProbeThreads, 0, stream>>>(static_cast<const probe_u32x4*>(p), n16, chunk, sink);
  return hipGetLastError();
}

}  // namespace mikv
