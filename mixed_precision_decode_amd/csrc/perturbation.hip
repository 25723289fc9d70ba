// Output-perturbation diagnostic: L = ||o - o_hat||_1 per head, in head
// space and after the head's output projection W_O,h.
//
// gist.science summary of arXiv 2502.03805 (CriticalKV), theoretical
// framework: replacing the full KV cache by a selected part perturbs the
// attention output by the L1 distance between the two outputs, and the bound
// of that perturbation involves the attention weights and the value states
// projected by W_O. o is the head's softmax attention over all T tokens;
// o_hat is the attention over the kept tokens with the softmax renormalized
// over them (an eviction), or an output the caller computed (a compressed
// cache, e.g. MiKV's mixed-precision decode attention).
//
// Kernels (HBM-bound streaming):
//   pert_mask_kernel   kept-token mask per head from the kept index lists;
//   pert_attn_kernel   one block per (split, head): streams K and V rows of
//                      its token range once, keeping two online softmaxes
//                      (all tokens, kept tokens); writes split partials;
//   pert_merge_kernel  one block per head: o, o_hat, delta = o - o_hat,
//                      ||delta||_1;
//   pert_proj_kernel   one block per (256 output columns, head):
//                      |delta . W_O,h[:, j]| summed over its columns;
//   pert_sum_kernel    the column blocks' sums per head.
#include <hip/hip_runtime.h>

#include <cfloat>

#include "common.hpp"
#include "kernels.hpp"

namespace mikv {

namespace {

constexpr int kPT = 256;                  // threads per block
constexpr float kPLog2e = 1.4426950408889634f;
constexpr int kProjCols = 256;            // output columns per projection block

typedef __amdgpu_buffer_rsrc_t PRsrc;
__device__ __forceinline__ PRsrc pert_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 pert_load16(PRsrc r, uint32_t off) {
  const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 2);
  return make_uint4(t[0], t[1], t[2], t[3]);
}

// Online softmax of one thread: running max (log2 units), sum, 8 channels.
struct PState {
  float m, l, a[8];
  __device__ __forceinline__ void init() {
    m = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = 0.0f;
  }
  __device__ __forceinline__ void add(float s, const float (&v)[8]) {
    if (s > m) {
      const float f = __builtin_amdgcn_exp2f(m - s);  // 0 when m was -inf
      l *= f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] *= f;
      m = s;
    }
    const float p = __builtin_amdgcn_exp2f(s - m);
    l += p;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] += p * v[i];
  }
};

__global__ __launch_bounds__(kPT) void pert_mask_kernel(const int32_t* __restrict__ keep, int n_keep, int T,
                                                         uint8_t* __restrict__ mask) {
  const int h = blockIdx.x;
  uint8_t* m = mask + static_cast<int64_t>(h) * T;
  for (int t = threadIdx.x; t < T; t += kPT) m[t] = 0;
  __syncthreads();
  const int32_t* kp = keep + static_cast<int64_t>(h) * n_keep;
  for (int i = threadIdx.x; i < n_keep; i += kPT) {
    const int t = kp[i];
    if (t >= 0 && t < T) m[t] = 1;  // indices outside [0, T) are ignored
  }
}

// Partials: part_ml [H][S][2] (max, sum) and part_o [H][S][2][D] (o sums),
// index 0 = all tokens, 1 = kept tokens.
template <int D>
__global__ __launch_bounds__(kPT) void pert_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* K,
                                                         const uint16_t* V, const uint8_t* __restrict__ mask,
                                                         int T, int chunk, float2* __restrict__ part_ml,
                                                         float* __restrict__ part_o) {
  constexpr int LPT = D / 8, SLOTS = kPT / LPT;
  const int split = blockIdx.x, h = blockIdx.y, S = gridDim.x;
  const int tid = threadIdx.x, lane = tid % LPT, slot = tid / LPT;
  const int t0 = split * chunk;
  const int t1 = min(T, t0 + chunk);
  const int nt = max(t1 - t0, 0);
  const int64_t rowb = (static_cast<int64_t>(h) * T + t0) * D;
  const PRsrc rk = pert_rsrc(K + rowb, static_cast<uint32_t>(nt) * D * 2);
  const PRsrc rv = pert_rsrc(V + rowb, static_cast<uint32_t>(nt) * D * 2);
  const uint8_t* mk = mask ? mask + static_cast<int64_t>(h) * T + t0 : nullptr;
  float qh[8];
  load8(q + static_cast<int64_t>(h) * D + lane * 8, qh);
  const float qs = kPLog2e / sqrtf(static_cast<float>(D));
#pragma unroll
  for (int i = 0; i < 8; ++i) qh[i] *= qs;
  PState all, kept;
  all.init();
  kept.init();
  for (int t = slot; t < nt; t += SLOTS) {
    const uint32_t off = static_cast<uint32_t>(t) * D * 2 + lane * 16;
    const uint4 kw = pert_load16(rk, off), vw = pert_load16(rv, off);
    const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w}, vv[4] = {vw.x, vw.y, vw.z, vw.w};
    float s = 0.0f, v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s += qh[2 * i] * lo_h(kk[i]) + qh[2 * i + 1] * hi_h(kk[i]);
      v[2 * i] = lo_h(vv[i]);
      v[2 * i + 1] = hi_h(vv[i]);
    }
    s = group_sum<LPT>(s);
    all.add(s, v);
    if (mk && mk[t]) kept.add(s, v);
  }
  // combine the slots: per state, max over slots, rescale, sum
  __shared__ float sm[2][SLOTS];
  __shared__ float so[2][SLOTS][D];
  __shared__ float sl[2][SLOTS];
  PState* st[2] = {&all, &kept};
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    if (lane == 0) {
      sm[w][slot] = st[w]->m;
      sl[w][slot] = st[w]->l;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) so[w][slot][lane * 8 + i] = st[w]->a[i];
  }
  __syncthreads();
  const int64_t pb = static_cast<int64_t>(h) * S + split;
  for (int i = tid; i < 2 * D; i += kPT) {
    const int w = i / D, c = i % D;
    float mx = -INFINITY;
    for (int j = 0; j < SLOTS; ++j) mx = fmaxf(mx, sm[w][j]);
    float o = 0.0f;
    for (int j = 0; j < SLOTS; ++j)
      if (sm[w][j] != -INFINITY) o += __builtin_amdgcn_exp2f(sm[w][j] - mx) * so[w][j][c];
    part_o[(pb * 2 + w) * D + c] = o;
  }
  if (tid < 2) {
    const int w = tid;
    float mx = -INFINITY;
    for (int j = 0; j < SLOTS; ++j) mx = fmaxf(mx, sm[w][j]);
    float L = 0.0f;
    for (int j = 0; j < SLOTS; ++j)
      if (sm[w][j] != -INFINITY) L += __builtin_amdgcn_exp2f(sm[w][j] - mx) * sl[w][j];
    part_ml[pb * 2 + w] = make_float2(mx, L);
  }
}

template <int D>
__global__ __launch_bounds__(D) void pert_merge_kernel(const float2* __restrict__ part_ml,
                                                        const float* __restrict__ part_o, int S,
                                                        const float* __restrict__ o_hat, float* __restrict__ o_out,
                                                        float* __restrict__ delta, float* __restrict__ L_head) {
  const int h = blockIdx.x, c = threadIdx.x;
  float res[2];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    if (w == 1 && o_hat) {
      res[1] = o_hat[static_cast<int64_t>(h) * D + c];
      continue;
    }
    float mx = -INFINITY;
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, part_ml[(static_cast<int64_t>(h) * S + s) * 2 + w].x);
    float L = 0.0f, o = 0.0f;
    for (int s = 0; s < S; ++s) {
      const float2 ml = part_ml[(static_cast<int64_t>(h) * S + s) * 2 + w];
      if (ml.x == -INFINITY) continue;
      const float f = __builtin_amdgcn_exp2f(ml.x - mx);
      L += f * ml.y;
      o += f * part_o[((static_cast<int64_t>(h) * S + s) * 2 + w) * D + c];
    }
    res[w] = o / L;
  }
  const float dl = res[0] - res[1];
  if (o_out) o_out[static_cast<int64_t>(h) * D + c] = res[0];
  delta[static_cast<int64_t>(h) * D + c] = dl;
  __shared__ float red[D];
  red[c] = fabsf(dl);
  __syncthreads();
  for (int k = D / 2; k > 0; k /= 2) {
    if (c < k) red[c] += red[c + k];
    __syncthreads();
  }
  if (c == 0) L_head[h] = red[0];
}

__global__ __launch_bounds__(kPT) void pert_proj_kernel(const float* __restrict__ delta,
                                                         const uint16_t* __restrict__ W, int D, int hidden,
                                                         float* __restrict__ part) {
  const int chunk = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  __shared__ float dl[128];
  __shared__ float red[kPT];
  if (tid < D) dl[tid] = delta[static_cast<int64_t>(h) * D + tid];
  __syncthreads();
  const int j = chunk * kProjCols + tid;
  float acc = 0.0f;
  if (j < hidden) {
    const uint16_t* w = W + static_cast<int64_t>(h) * D * hidden + j;
    for (int c = 0; c < D; ++c) acc += dl[c] * h2f(w[static_cast<int64_t>(c) * hidden]);
  }
  red[tid] = fabsf(acc);
  __syncthreads();
  for (int k = kPT / 2; k > 0; k /= 2) {
    if (tid < k) red[tid] += red[tid + k];
    __syncthreads();
  }
  if (tid == 0) part[static_cast<int64_t>(h) * gridDim.x + chunk] = red[0];
}

__global__ __launch_bounds__(kWave) void pert_sum_kernel(const float* __restrict__ part, int nchunk,
                                                          float* __restrict__ L_proj) {
  const int h = blockIdx.x;
  float s = 0.0f;
  for (int i = threadIdx.x; i < nchunk; i += kWave) s += part[static_cast<int64_t>(h) * nchunk + i];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (threadIdx.x == 0) L_proj[h] = s;
}

inline size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

int perturbation_splits(int H, int T) {
  int s = (1024 + H - 1) / H;   // about 1024 blocks in all
  const int per = (T + 255) / 256;  // at least 256 tokens per split
  if (s > per) s = per;
  return s < 1 ? 1 : s;
}

size_t perturbation_ws_bytes(int H, int T, int d, int hidden) {
  const size_t S = perturbation_splits(H, T);
  const size_t nchunk = (hidden + kProjCols - 1) / kProjCols;
  return al256(static_cast<size_t>(H) * T) + al256(H * S * 2 * sizeof(float2)) +
         al256(H * S * 2 * d * sizeof(float)) + al256(static_cast<size_t>(H) * d * sizeof(float)) +
         al256(H * nchunk * sizeof(float));
}

hipError_t launch_perturbation(const uint16_t* q, const uint16_t* K, const uint16_t* V, const uint16_t* W,
                               const int32_t* keep, int n_keep, const float* o_hat, int H, int T, int d,
                               int hidden, float* o, float* delta_out, float* L_head, float* L_proj,
                               void* ws, hipStream_t stream) {
  const int S = perturbation_splits(H, T);
  const int chunk = (T + S - 1) / S;
  const int nchunk = (hidden + kProjCols - 1) / kProjCols;
  char* w = static_cast<char*>(ws);
  uint8_t* mask = reinterpret_cast<uint8_t*>(w);
  w += al256(static_cast<size_t>(H) * T);
  float2* part_ml = reinterpret_cast<float2*>(w);
  w += al256(static_cast<size_t>(H) * S * 2 * sizeof(float2));
  float* part_o = reinterpret_cast<float*>(w);
  w += al256(static_cast<size_t>(H) * S * 2 * d * sizeof(float));
  float* delta = delta_out ? delta_out : reinterpret_cast<float*>(w);
  w += al256(static_cast<size_t>(H) * d * sizeof(float));
  float* part = reinterpret_cast<float*>(w);
  if (keep) {
    pert_mask_kernel<<<H, kPT, 0, stream>>>(keep, n_keep, T, mask);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(static_cast<unsigned>(S), static_cast<unsigned>(H));
  if (d == 128) {
    pert_attn_kernel<128><<<grid, kPT, 0, stream>>>(q, K, V, keep ? mask : nullptr, T, chunk, part_ml, part_o);
    pert_merge_kernel<128><<<H, 128, 0, stream>>>(part_ml, part_o, S, keep ? nullptr : o_hat, o, delta, L_head);
  } else {
    pert_attn_kernel<64><<<grid, kPT, 0, stream>>>(q, K, V, keep ? mask : nullptr, T, chunk, part_ml, part_o);
    pert_merge_kernel<64><<<H, 64, 0, stream>>>(part_ml, part_o, S, keep ? nullptr : o_hat, o, delta, L_head);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  pert_proj_kernel<<<dim3(static_cast<unsigned>(nchunk), static_cast<unsigned>(H)), kPT, 0, stream>>>(
      delta, W, d, hidden, part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  pert_sum_kernel<<<H, kWave, 0, stream>>>(part, nchunk, L_proj);
  return hipGetLastError();
}

}  // namespace mikv
