// Block-wide top-m selection by (key descending, index ascending) with
// 32-bit order-preserving keys, and block prefix sums.
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

// Exclusive prefix sum of an int over the block (NT threads), in thread
// order. Every thread must call it; *total receives the block sum.
template <int NT>
__device__ __forceinline__ int block_scan_add(int v, int* total) {
  constexpr int NWV = NT / kWave;
  __shared__ int s_w[NWV];
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) s_w[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) {
    off += (i < w) ? s_w[i] : 0;
    tot += s_w[i];
  }
  *total = tot;
  __syncthreads();
  return off + incl - v;
}

// Radix select (4 passes of 8 bits, most significant first) of the m-th
// largest key among the elements i in [0, n) for which keyfn(i, &key) is
// true, by a block of NT threads. On return, on every thread: *tau is that
// key and *need the number of elements equal to *tau that belong to the top
// m (the lowest-index ones); elements with key > *tau all belong to it.
// Requires 1 <= m <= count. Each wave counts into its own histogram (keys
// such as probabilities share few top bytes, so one shared histogram
// serialises the atomics); the histograms are summed before the digit search.
//
// When n <= NT * KPT, each thread first loads its keys (elements tid,
// tid + NT, ...) into registers with every load in flight, and the four
// passes count from registers; otherwise each pass reads the keys again.
template <int NT = 256, int KPT = 0, class KeyFn>
__device__ void block_radix_topm(int n, int m, KeyFn keyfn, uint32_t* tau, int* need) {
  constexpr int NWV = NT / kWave;
  __shared__ uint32_t hist[NWV][256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const int tid = threadIdx.x, wv = tid / kWave;
  uint32_t prefix = 0, mask = 0;
  int nd = m;
  constexpr int KC = KPT > 0 ? KPT : 1;
  static_assert(KC <= 32, "validity of the cached keys is one 32-bit mask");
  const bool cached = KPT > 0 && n <= NT * KPT;
  uint32_t kc[KC];
  uint32_t kvalid = 0;
  if (cached) {
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const int i = tid + j * NT;
      kc[j] = 0;
      if (i < n && keyfn(i, &kc[j])) kvalid |= 1u << j;
    }
  }
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < NWV * 256; i += NT) (&hist[0][0])[i] = 0;
    __syncthreads();
    if (cached) {
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (((kvalid >> j) & 1u) && (kc[j] & mask) == prefix) atomicAdd(&hist[wv][(kc[j] >> shift) & 0xFFu], 1u);
    } else {
      for (int i = tid; i < n; i += NT) {
        uint32_t key;
        if (keyfn(i, &key) && (key & mask) == prefix) atomicAdd(&hist[wv][(key >> shift) & 0xFFu], 1u);
      }
    }
    __syncthreads();
    if (NWV > 1) {
      for (int dg = tid; dg < 256; dg += NT) {
        uint32_t t = hist[0][dg];
#pragma unroll
        for (int w = 1; w < NWV; ++w) t += hist[w][dg];
        hist[0][dg] = t;
      }
      __syncthreads();
    }
    if (tid < kWave) {
      // lane owns digits 255-4*lane .. 252-4*lane (descending); find the
      // first digit (from the top) where the running count reaches nd.
      int c[4];
      int sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = static_cast<int>(hist[0][255 - 4 * tid - j]); sum += c[j]; }
      // inclusive scan of lane sums across the wave
      const int incl = wave_incl_scan(sum);
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
