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
//   pert_attn_kernel   one block per (split, head): marks its range's kept
//                      tokens in an LDS bitmap from the head's kept index
//                      list, then streams K and V rows of the range once,
//                      keeping two online softmaxes (all tokens, kept
//                      tokens); writes split partials;
//   pert_out_kernel    one block per (512 output columns, head): combines
//                      the head's partials into o, o_hat and delta = o -
//                      o_hat (column block 0 writes them and ||delta||_1),
//                      then |delta . W_O,h[:, j]| summed over its columns,
//                      W_O read in 16-byte rows by 4 row groups;
//   pert_sum_kernel    the column blocks' sums per head.
#include <hip/hip_runtime.h>

#include <cfloat>

#include "common.hpp"
#include "kernels.hpp"

namespace mikv {

namespace {

constexpr int kPT = 256;                  // threads per block
constexpr float kPLog2e = 1.4426950408889634f;
constexpr int kProjCols = 512;            // output columns per projection block (64 x 8)
constexpr int kMaxChunk = 65536;          // tokens per split at most (LDS bitmap of 8 KB)

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

// Partials: part_ml [H][S][2] (max, sum) and part_o [H][S][2][D] (o sums),
// index 0 = all tokens, 1 = kept tokens.
template <int D>
__global__ __launch_bounds__(kPT) void pert_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* K,
                                                         const uint16_t* V, const int32_t* __restrict__ keep,
                                                         int n_keep, int T, int chunk, float2* __restrict__ part_ml,
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
  // kept tokens of the range as a bitmap (indices outside [0, T) ignored)
  __shared__ uint32_t kept_bits[kMaxChunk / 32];
  if (keep) {  // uniform
    const int nw = (nt + 31) / 32;
    for (int i = tid; i < nw; i += kPT) kept_bits[i] = 0u;
    __syncthreads();
    const int32_t* kp = keep + static_cast<int64_t>(h) * n_keep;
    for (int i = tid; i < n_keep; i += kPT) {
      const int t = kp[i] - t0;
      if (t >= 0 && t < nt) atomicOr(&kept_bits[t / 32], 1u << (t % 32));
    }
    __syncthreads();
  }
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
    if (keep && ((kept_bits[t / 32] >> (t % 32)) & 1u)) kept.add(s, v);
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

// o, o_hat and delta of head h for its D channels (every block of the head
// recomputes them from the split partials, which stay in L2), then the
// projection of delta onto the block's 512 columns of W_O,h: 64 column
// groups of 8 x 4 row groups of D/4 rows, 16-byte loads (hidden a multiple
// of 8); the row groups' column sums are added before |.|.
template <int D, bool VEC>
__global__ __launch_bounds__(kPT) void pert_out_kernel(const float2* __restrict__ part_ml,
                                                        const float* __restrict__ part_o, int S,
                                                        const float* __restrict__ o_hat, const uint16_t* W,
                                                        int hidden, float* __restrict__ o_out,
                                                        float* __restrict__ delta, float* __restrict__ L_head,
                                                        float* __restrict__ part) {
  const int chunk = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  __shared__ float sM[2], sIL[2];
  __shared__ float dl[D];
  __shared__ float red[kPT][8];
  // (1) per state: max and reciprocal sum over the splits, one wave each
  {
    const int wave = tid / kWave, ln = tid % kWave;
    if (wave < 2 && !(wave == 1 && o_hat)) {
      const float2* ml = part_ml + static_cast<int64_t>(h) * S * 2 + wave;
      float mx = -INFINITY;
      for (int s = ln; s < S; s += kWave) mx = fmaxf(mx, ml[2 * s].x);
      mx = wave_max(mx);
      float L = 0.0f;
      for (int s = ln; s < S; s += kWave) {
        const float2 v = ml[2 * s];
        if (v.x != -INFINITY) L += __builtin_amdgcn_exp2f(v.x - mx) * v.y;
      }
      L = wave_sum(L);
      if (ln == 0) {
        sM[wave] = mx;
        sIL[wave] = 1.0f / L;
      }
    }
  }
  __syncthreads();
  // (2) o and o_hat per channel: thread (w, c) for w = tid / D
  if (tid < 2 * D) {
    const int w = tid / D, c = tid % D;
    float res;
    if (w == 1 && o_hat) {
      res = o_hat[static_cast<int64_t>(h) * D + c];
    } else {
      const float mx = sM[w];
      const float2* ml = part_ml + static_cast<int64_t>(h) * S * 2 + w;
      const float* po = part_o + (static_cast<int64_t>(h) * S * 2 + w) * D + c;
      float o = 0.0f;
#pragma unroll 8
      for (int s = 0; s < S; ++s) {
        const float2 v = ml[2 * s];
        const float x = po[static_cast<int64_t>(s) * 2 * D];
        if (v.x != -INFINITY) o += __builtin_amdgcn_exp2f(v.x - mx) * x;
      }
      res = o * sIL[w];
    }
    red[tid][0] = res;
  }
  __syncthreads();
  if (tid < D) {
    const float o = red[tid][0], oh = red[D + tid][0];
    const float d = o - oh;
    dl[tid] = d;
    if (chunk == 0) {
      if (o_out) o_out[static_cast<int64_t>(h) * D + tid] = o;
      delta[static_cast<int64_t>(h) * D + tid] = d;
    }
  }
  __syncthreads();
  if (chunk == 0 && tid < kWave) {
    float a = 0.0f;
    for (int c = tid; c < D; c += kWave) a += fabsf(dl[c]);
    a = wave_sum(a);
    if (tid == 0) L_head[h] = a;
  }
  // (3) projection: column group cg (8 columns), row group rg (D/4 rows)
  constexpr int RPG = D / 4;
  const int cg = tid % 64, rg = tid / 64;
  const int j0 = chunk * kProjCols + cg * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  const uint16_t* wh = W + static_cast<int64_t>(h) * D * hidden;
  if constexpr (VEC) {
    // a column group lies wholly inside or outside [0, hidden) (hidden is a
    // multiple of 8); groups outside add nothing (their addresses would be
    // the next row's columns)
    if (j0 < hidden) {
    const PRsrc rw = pert_rsrc(wh, static_cast<uint32_t>(D) * hidden * 2);
    uint4 wv[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r)
      wv[r] = pert_load16(rw, static_cast<uint32_t>((rg * RPG + r) * hidden + j0) * 2);
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
      const float dv = dl[rg * RPG + r];
      const uint32_t ww[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += dv * lo_h(ww[i]);
        acc[2 * i + 1] += dv * hi_h(ww[i]);
      }
    }
    }
  } else {
    for (int r = 0; r < RPG; ++r) {
      const float dv = dl[rg * RPG + r];
      const uint16_t* wr = wh + static_cast<int64_t>(rg * RPG + r) * hidden;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (j0 + e < hidden) acc[e] += dv * h2f(wr[j0 + e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tid][e] = acc[e];
  __syncthreads();
  float colabs = 0.0f;
  if (tid < 64) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      colabs += fabsf(red[tid][e] + red[64 + tid][e] + red[128 + tid][e] + red[192 + tid][e]);
  }
  if (tid < kWave) {
    colabs = wave_sum(colabs);
    if (tid == 0) part[static_cast<int64_t>(h) * gridDim.x + chunk] = colabs;
  }
}

__global__ __launch_bounds__(kWave) void pert_sum_kernel(const float* __restrict__ part, int nchunk,
                                                          float* __restrict__ L_proj) {
  const int h = blockIdx.x;
  float s = 0.0f;
  for (int i = threadIdx.x; i < nchunk; i += kWave) s += part[static_cast<int64_t>(h) * nchunk + i];
  s = wave_sum(s);
  if (threadIdx.x == 0) L_proj[h] = s;
}

inline size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

int perturbation_splits(int H, int T) {
  int s = (1024 + H - 1) / H;   // about 1024 blocks in all
  const int per = (T + 255) / 256;  // at least 256 tokens per split
  if (s > per) s = per;
  const int fit = (T + kMaxChunk - 1) / kMaxChunk;  // the kept bitmap of a split fits LDS
  if (s < fit) s = fit;
  return s < 1 ? 1 : s;
}

size_t perturbation_ws_bytes(int H, int T, int d, int hidden) {
  const size_t S = perturbation_splits(H, T);
  const size_t nchunk = (hidden + kProjCols - 1) / kProjCols;
  return al256(H * S * 2 * sizeof(float2)) + al256(H * S * 2 * d * sizeof(float)) +
         al256(static_cast<size_t>(H) * d * sizeof(float)) + al256(H * nchunk * sizeof(float));
}

hipError_t launch_perturbation(const uint16_t* q, const uint16_t* K, const uint16_t* V, const uint16_t* W,
                               const int32_t* keep, int n_keep, const float* o_hat, int H, int T, int d,
                               int hidden, float* o, float* delta_out, float* L_head, float* L_proj,
                               void* ws, hipStream_t stream) {
  const int S = perturbation_splits(H, T);
  const int chunk = (T + S - 1) / S;
  const int nchunk = (hidden + kProjCols - 1) / kProjCols;
  char* w = static_cast<char*>(ws);
  float2* part_ml = reinterpret_cast<float2*>(w);
  w += al256(static_cast<size_t>(H) * S * 2 * sizeof(float2));
  float* part_o = reinterpret_cast<float*>(w);
  w += al256(static_cast<size_t>(H) * S * 2 * d * sizeof(float));
  float* delta = delta_out ? delta_out : reinterpret_cast<float*>(w);
  w += al256(static_cast<size_t>(H) * d * sizeof(float));
  float* part = reinterpret_cast<float*>(w);
  const dim3 grid(static_cast<unsigned>(S), static_cast<unsigned>(H));
  const dim3 ogrid(static_cast<unsigned>(nchunk), static_cast<unsigned>(H));
  const float* oh = keep ? nullptr : o_hat;
  // 16-byte rows of W_O: hidden a multiple of 8 and W_O 16-byte aligned
  const bool vec = hidden % 8 == 0 && (reinterpret_cast<uintptr_t>(W) & 15u) == 0;
  if (d == 128) {
    pert_attn_kernel<128><<<grid, kPT, 0, stream>>>(q, K, V, keep, n_keep, T, chunk, part_ml, part_o);
    if (vec) pert_out_kernel<128, true><<<ogrid, kPT, 0, stream>>>(part_ml, part_o, S, oh, W, hidden, o, delta, L_head, part);
    else pert_out_kernel<128, false><<<ogrid, kPT, 0, stream>>>(part_ml, part_o, S, oh, W, hidden, o, delta, L_head, part);
  } else {
    pert_attn_kernel<64><<<grid, kPT, 0, stream>>>(q, K, V, keep, n_keep, T, chunk, part_ml, part_o);
    if (vec) pert_out_kernel<64, true><<<ogrid, kPT, 0, stream>>>(part_ml, part_o, S, oh, W, hidden, o, delta, L_head, part);
    else pert_out_kernel<64, false><<<ogrid, kPT, 0, stream>>>(part_ml, part_o, S, oh, W, hidden, o, delta, L_head, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  pert_sum_kernel<<<H, kWave, 0, stream>>>(part, nchunk, L_proj);
  return hipGetLastError();
}

}  // namespace mikv
