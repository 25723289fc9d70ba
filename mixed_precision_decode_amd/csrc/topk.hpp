// Block-wide (256 threads) top-m selection by (key descending, index
// ascending) with 32-bit order-preserving keys, and block prefix sums.
#pragma once

#include "common.hpp"

namespace mikv {

// Exclusive prefix sum of a 0/1 flag over the block, in thread order.
// Every thread of the block must call it. *total receives the block sum.
__device__ __forceinline__ int block_prefix(int flag, int* total) {
  __shared__ int s_w[4];
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const unsigned long long m = __ballot(flag);
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) s_w[w] = __popcll(m);
  __syncthreads();
  int off = 0;
  for (int i = 0; i < w; ++i) off += s_w[i];
  *total = s_w[0] + s_w[1] + s_w[2] + s_w[3];
  __syncthreads();
  return off + in_wave;
}

// Radix select (4 passes of 8 bits, most significant first) of the m-th
// largest key among the elements i in [0, n) for which keyfn(i, &key) is
// true. On return, on every thread: *tau is that key and *need the number of
// elements equal to *tau that belong to the top m (the lowest-index ones);
// elements with key > *tau all belong to it. Requires 1 <= m <= count.
template <class KeyFn>
__device__ void block_radix_topm(int n, int m, KeyFn keyfn, uint32_t* tau, int* need) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  int nd = m;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      uint32_t key;
      if (keyfn(i, &key) && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFFu], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      // lane owns digits 255-4*lane .. 252-4*lane (descending); find the
      // first digit (from the top) where the running count reaches nd.
      int c[4];
      int sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = static_cast<int>(hist[255 - 4 * tid - j]); sum += c[j]; }
      // inclusive scan of lane sums across the wave
      int incl = sum;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (tid >= off) incl += o;
      }
      const int excl = incl - sum;
      const bool hit = excl < nd && incl >= nd;
      if (hit) {
        int cum = excl, dsel = 255 - 4 * tid;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum + c[j] >= nd) { dsel = 255 - 4 * tid - j; break; }
          cum += c[j];
        }
        s_need = nd - cum;
        s_prefix = prefix | (static_cast<uint32_t>(dsel) << shift);
      }
    }
    __syncthreads();
    nd = s_need;
    prefix = s_prefix;
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  *tau = prefix;
  *need = nd;
}

}  // namespace mikv
