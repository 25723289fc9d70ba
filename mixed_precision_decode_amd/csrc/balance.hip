// Channel balancer b = sqrt(max|q| / max|k|) per sequence, kv head, channel,
// and the balanced keys kb = fp16(k * b).
//
// velog notes "No Token Left Behind ...", Key contributions 2)
// (Outlier-aware): balancer equation over the prefill tokens, and the k-hat
// equation (keys multiplied by b before quantization). paperlayer summary of
// arXiv 2402.18096, section 3.2: computed once at prefill.
//
// Pass 1 streams the prompt's q rows (all query heads of the kv head) and k
// rows in chunks and writes per-chunk channel maxima; pass 2 reduces the
// chunk maxima and evaluates b; pass 3 (optional) writes kb. All passes are
// HBM-bound; the maxima are exact (|fp16| compares).
#include "common.hpp"
#include "kernels.hpp"

namespace mikv {

constexpr int kBalChunkRows = 256;

static inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

template <int D>
__global__ __launch_bounds__(256) void balance_partial_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              int rep, int T, int nqc, int nkc,
                                                              float* __restrict__ part) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int nch = nqc + nkc;
  const int unit = blockIdx.x / nch;
  const int ch = blockIdx.x % nch;
  const uint16_t* base;
  int nrows, r0;
  if (ch < nqc) {
    // q rows of the group: heads g*rep .. g*rep+rep-1 are contiguous.
    base = q + static_cast<int64_t>(unit) * rep * T * D;
    nrows = rep * T;
    r0 = ch * kBalChunkRows;
  } else {
    base = k + static_cast<int64_t>(unit) * T * D;
    nrows = T;
    r0 = (ch - nqc) * kBalChunkRows;
  }
  const int r1 = min(nrows, r0 + kBalChunkRows);
  const int lane = threadIdx.x % LPR;
  float m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = 0.0f;
  for (int r = r0 + threadIdx.x / LPR; r < r1; r += RPB) {
    float x[8];
    load8(base + static_cast<int64_t>(r) * D + lane * 8, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(x[i]));
  }
  __shared__ float red[RPB][D];
#pragma unroll
  for (int i = 0; i < 8; ++i) red[threadIdx.x / LPR][lane * 8 + i] = m[i];
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += 256) {
    float v = 0.0f;
    for (int s = 0; s < RPB; ++s) v = fmaxf(v, red[s][c]);
    part[static_cast<int64_t>(blockIdx.x) * D + c] = v;
  }
}

// One block per (sequence, kv head): 1024 / D groups of threads take
// interleaved chunk subsets, with several loads in flight per thread, and
// combine through LDS (a long prompt has hundreds of chunks).
constexpr int kFinThreads = 1024;
template <int D>
__global__ __launch_bounds__(kFinThreads) void balance_finalize_kernel(const float* __restrict__ part,
                                                                      int units, int nqc, int nkc,
                                                                      float* __restrict__ b) {
  constexpr int NG = kFinThreads / D;
  __shared__ float red[2][NG][D];
  const int unit = blockIdx.x;
  const int c = threadIdx.x % D, grp = threadIdx.x / D;
  const float* p = part + static_cast<int64_t>(unit) * (nqc + nkc) * D + c;
  auto chunk_max = [&](int j0, int j1) {
    float m0 = 0.0f, m1 = 0.0f, m2 = 0.0f, m3 = 0.0f;
    int j = j0 + grp;
    for (; j + 3 * NG < j1; j += 4 * NG) {
      m0 = fmaxf(m0, p[static_cast<int64_t>(j) * D]);
      m1 = fmaxf(m1, p[static_cast<int64_t>(j + NG) * D]);
      m2 = fmaxf(m2, p[static_cast<int64_t>(j + 2 * NG) * D]);
      m3 = fmaxf(m3, p[static_cast<int64_t>(j + 3 * NG) * D]);
    }
    for (; j < j1; j += NG) m0 = fmaxf(m0, p[static_cast<int64_t>(j) * D]);
    return fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
  };
  red[0][grp][c] = chunk_max(0, nqc);
  red[1][grp][c] = chunk_max(nqc, nqc + nkc);
  __syncthreads();
  if (grp == 0) {
    float mq = 0.0f, mk = 0.0f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      mq = fmaxf(mq, red[0][i][c]);
      mk = fmaxf(mk, red[1][i][c]);
    }
    float r = 1.0f;
    if (mq != 0.0f && mk != 0.0f) r = sqrtf(mq / mk);
    b[static_cast<int64_t>(unit) * D + c] = r;
  }
}

template <int D>
__global__ __launch_bounds__(256) void balance_keys_kernel(const uint16_t* __restrict__ k,
                                                           const float* __restrict__ b, int T,
                                                           int64_t n_rows,
                                                           uint16_t* __restrict__ kb) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int lane = threadIdx.x % LPR;
  const int64_t step = static_cast<int64_t>(gridDim.x) * RPB;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR; r < n_rows; r += step) {
    const int64_t unit = r / T;
    float x[8];
    load8(k + r * D + lane * 8, x);
    const float* bb = b + unit * D + lane * 8;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = f2h(mul_rn(x[2 * i], bb[2 * i]));
      const uint32_t hi = f2h(mul_rn(x[2 * i + 1], bb[2 * i + 1]));
      w[i] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(kb + r * D + lane * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

size_t balance_ws_bytes(int batch, int hkv, int rep, int d, int T) {
  const int nqc = ceil_div(rep * T, kBalChunkRows);
  const int nkc = ceil_div(T, kBalChunkRows);
  return static_cast<size_t>(batch) * hkv * (nqc + nkc) * d * sizeof(float);
}

template <int D>
static hipError_t launch_bal(int batch, int hq, int hkv, int T, const uint16_t* q,
                             const uint16_t* k, float* b, uint16_t* kb, void* ws,
                             hipStream_t stream) {
  const int rep = hq / hkv;
  const int units = batch * hkv;
  const int nqc = ceil_div(rep * T, kBalChunkRows);
  const int nkc = ceil_div(T, kBalChunkRows);
  float* part = static_cast<float*>(ws);
  if (nqc + nkc > 0) {
    balance_partial_kernel<D><<<units * (nqc + nkc), 256, 0, stream>>>(q, k, rep, T, nqc, nkc, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  balance_finalize_kernel<D><<<units, kFinThreads, 0, stream>>>(part, units, nqc, nkc, b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (kb && T > 0) {
    const int64_t n_rows = static_cast<int64_t>(units) * T;
    constexpr int RPB = 256 / (D / 8);
    int64_t blocks = (n_rows + RPB - 1) / RPB;
    if (blocks > 65536) blocks = 65536;
    balance_keys_kernel<D><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(k, b, T, n_rows, kb);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_balance(int batch, int hq, int hkv, int d, int T, const uint16_t* q,
                          const uint16_t* k, float* b, uint16_t* kb, void* ws,
                          hipStream_t stream) {
  if (d == 128) return launch_bal<128>(batch, hq, hkv, T, q, k, b, kb, ws, stream);
  if (d == 64) return launch_bal<64>(batch, hq, hkv, T, q, k, b, kb, ws, stream);
  return hipErrorInvalidValue;
}

}  // namespace mikv
