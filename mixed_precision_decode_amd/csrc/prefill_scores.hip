// Prompt heavy-hitter scores acc0 on the GPU.
//
// paperlayer summary of arXiv 2402.18096, section 5 and velog notes "No
// Token Left Behind ...", Key contributions 1): the important set is chosen
// by accumulated attention (H2O). Over the prompt, the score of token t sums
// the causal softmax weights P[i][t] = softmax_t'<=i(q_i . k_t' / sqrt(d))
// over the queries i >= t and over the query heads of t's kv head; the decode
// steps keep adding to the same sums.
//
// Two passes, both on MFMA (the T x T score matrix of a head is a dense
// contraction over d), computing S^T = K Q^T tile by tile with
// v_mfma_f32_32x32x16_f16 (fp16 in, fp32 accumulation). In that orientation
// a lane's 16 accumulator registers are 16 key rows of ONE query column, so
// the softmax statistics of a query need no cross-lane work per tile.
//   pass 1 (rowstat)  one wave per (sequence, query head, 32 queries); the
//                     queries' rows are the held B operand, the causal key
//                     tiles stream through the A operand; each lane keeps an
//                     online (max, sum) of its column; the two lanes of a
//                     column combine at the end -> (M_i, 1/L_i) in log2 units.
//   pass 2 (colsum)   one wave per (sequence, kv head, 32 keys); the keys'
//                     rows are the held A operand; every query tile at or
//                     after the diagonal of every head of the group streams
//                     through the B operand; p = exp2(s - M_i) / L_i is
//                     summed per key row in registers, then across the 32
//                     lanes that share the rows -> acc0.
// The two passes compute bit-identical scores (same operands, same MFMA
// sequence), so every p <= 1. No LDS, no atomics, no barriers: each wave
// owns its outputs. Blocks with the most tiles are dispatched first.
#include <cfloat>

#include "common.hpp"
#include "kernels.hpp"

namespace mikv {

namespace {

typedef _Float16 ps_half8 __attribute__((ext_vector_type(8)));
typedef float ps_floatx16 __attribute__((ext_vector_type(16)));

constexpr int kPsWaves = 4;                 // waves per block
constexpr int kPsThreads = kPsWaves * kWave;
constexpr int kPsTile = 32;                 // rows (keys or queries) per wave
constexpr int kPsBlockRows = kPsWaves * kPsTile;
constexpr float kPsLog2e = 1.4426950408889634f;

// MFMA 32x32x16 operand layout (lane l): A[l%32][8*(l/32) + 0..7],
// B[8*(l/32) + 0..7][l%32], D register r: row 8*(r/4) + 4*(l/32) + r%4,
// column l%32. For S^T = K Q^T both operands are 16-byte slices of rows:
// lane l reads row (l%32) of its tile at channels 16*ks + 8*(l/32) .. +7.
template <int D>
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ base, int row, ps_half8 (&f)[D / 16]) {
  const int lane = threadIdx.x % kWave;
  const uint16_t* p = base + static_cast<int64_t>(row) * D + 8 * (lane / 32);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    f[ks] = __builtin_bit_cast(ps_half8, *reinterpret_cast<const uint4*>(p + 16 * ks));
}

template <int D>
__device__ __forceinline__ ps_floatx16 scores(const ps_half8 (&a)[D / 16], const ps_half8 (&b)[D / 16]) {
  ps_floatx16 c = {};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ks], b[ks], c, 0, 0, 0);
  return c;
}

// key row of accumulator register r within a 32-row tile
__device__ __forceinline__ int row_of(int r, int lane) { return 8 * (r / 4) + 4 * (lane / 32) + (r % 4); }

template <int D>
__global__ __launch_bounds__(kPsThreads) void ps_rowstat_kernel(const uint16_t* __restrict__ q,
                                                                  const uint16_t* __restrict__ k, int hq,
                                                                  int hkv, int T, int nh, int nib,
                                                                  float2* __restrict__ stat) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  // the last query blocks (most key tiles) first
  const int ib = nib - 1 - static_cast<int>(blockIdx.x) / nh;
  const int nhi = static_cast<int>(blockIdx.x) % nh;  // n * hq + h
  const int n = nhi / hq, h = nhi % hq;
  const int g = h / (hq / hkv);
  const int i0 = ib * kPsBlockRows + wave * kPsTile;
  if (i0 >= T) return;
  const int i = i0 + lane % 32;  // this lane's query column
  const uint16_t* qb = q + static_cast<int64_t>(nhi) * T * D;
  const uint16_t* kb = k + (static_cast<int64_t>(n) * hkv + g) * T * D;
  ps_half8 bq[D / 16];
  load_rows<D>(qb, min(i, T - 1), bq);
  const float c = kPsLog2e / sqrtf(static_cast<float>(D));
  const int last = min(i0 + kPsTile - 1, T - 1);  // last key any lane of the wave needs
  const int ntiles = last / kPsTile + 1;
  float m = -INFINITY, l = 0.0f;
  ps_half8 ka[D / 16], kn[D / 16] = {};
  load_rows<D>(kb, min(lane % 32, T - 1), ka);
  for (int tt = 0; tt < ntiles; ++tt) {
    const int t0 = tt * kPsTile;
    if (tt + 1 < ntiles) load_rows<D>(kb, min(t0 + kPsTile + lane % 32, T - 1), kn);
    const ps_floatx16 s = scores<D>(ka, bq);
    float sv[16];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + row_of(r, lane);
      sv[r] = (t <= i) ? s[r] * c : -INFINITY;  // causal; t <= i < T keeps t in range
      mt = fmaxf(mt, sv[r]);
    }
    if (mt > m) {
      l *= exp2f(m - mt);  // 0 while m is -inf
      m = mt;
    }
    const float mref = fmaxf(m, -FLT_MAX);
#pragma unroll
    for (int r = 0; r < 16; ++r) l += exp2f(sv[r] - mref);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) ka[ks] = kn[ks];
  }
  // lanes l and l + 32 hold the two halves of column i's key rows
  const float mo = shfl_xor_f(m, 32), lo = shfl_xor_f(l, 32);
  const float M = fmaxf(m, mo);  // finite: key t = i is in lane l or l + 32
  const float L = l * exp2f(m - M) + lo * exp2f(mo - M);
  if (lane < 32 && i < T) stat[static_cast<int64_t>(nhi) * T + i] = make_float2(M, 1.0f / L);
}

template <int D>
__global__ __launch_bounds__(kPsThreads) void ps_colsum_kernel(const uint16_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ k, int hq,
                                                                 int hkv, int T, int ng,
                                                                 const float2* __restrict__ stat,
                                                                 float* __restrict__ acc0) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  // the first key blocks (most query tiles) first
  const int tb = static_cast<int>(blockIdx.x) / ng;
  const int ngi = static_cast<int>(blockIdx.x) % ng;  // n * hkv + g
  const int n = ngi / hkv, g = ngi % hkv;
  const int rep = hq / hkv;
  const int t0 = tb * kPsBlockRows + wave * kPsTile;
  if (t0 >= T) return;
  const uint16_t* kb = k + static_cast<int64_t>(ngi) * T * D;
  ps_half8 ka[D / 16];
  load_rows<D>(kb, min(t0 + lane % 32, T - 1), ka);
  const float c = kPsLog2e / sqrtf(static_cast<float>(D));
  float col[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) col[r] = 0.0f;
  const int first = t0 / kPsTile, ntiles = (T - 1) / kPsTile + 1;
  const int per_head = ntiles - first;
  const int total = rep * per_head;
  // iteration j: head h = g*rep + j / per_head, query tile first + j % per_head
  auto src = [&](int j, const uint16_t*& qb, const float2*& st, int& i) {
    const int h = g * rep + j / per_head;
    const int nhi = n * hq + h;
    i = (first + j % per_head) * kPsTile + lane % 32;
    qb = q + static_cast<int64_t>(nhi) * T * D;
    st = stat + static_cast<int64_t>(nhi) * T;
  };
  ps_half8 bq[D / 16], bn[D / 16] = {};
  float2 ms, mn = make_float2(0.0f, 0.0f);
  {
    const uint16_t* qb;
    const float2* st;
    int i;
    src(0, qb, st, i);
    load_rows<D>(qb, min(i, T - 1), bq);
    ms = st[min(i, T - 1)];
  }
  for (int j = 0; j < total; ++j) {
    const uint16_t* qb;
    const float2* st;
    int i, in;
    src(j, qb, st, i);
    if (j + 1 < total) {
      const uint16_t* qn;
      const float2* sn;
      src(j + 1, qn, sn, in);
      load_rows<D>(qn, min(in, T - 1), bn);
      mn = sn[min(in, T - 1)];
    }
    const ps_floatx16 s = scores<D>(ka, bq);
    // a query past the prompt contributes nothing: exp2(-inf) * 0
    const float M = (i < T) ? ms.x : INFINITY;
    const float IL = (i < T) ? ms.y : 0.0f;
    if ((i & ~(kPsTile - 1)) == t0) {  // diagonal tile: causal mask
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + row_of(r, lane);
        col[r] += (t <= i) ? exp2f(s[r] * c - M) * IL : 0.0f;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) col[r] += exp2f(s[r] * c - M) * IL;
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) bq[ks] = bn[ks];
    ms = mn;
  }
  // sum over the 32 query columns of the lanes that share l / 32
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float v = col[r];
    v += shfl_xor_f(v, 1);
    v += shfl_xor_f(v, 2);
    v += shfl_xor_f(v, 4);
    v += shfl_xor_f(v, 8);
    v += shfl_xor_f(v, 16);
    col[r] = v;
  }
  if (lane % 32 == 0) {
    float* out = acc0 + static_cast<int64_t>(ngi) * T;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + row_of(r, lane);
      if (t < T) out[t] = col[r];
    }
  }
}

}  // namespace

size_t prefill_scores_ws_bytes(int batch, int hq, int T) {
  return static_cast<size_t>(batch) * hq * T * sizeof(float2);
}

hipError_t launch_prefill_scores(int batch, int hq, int hkv, int d, int T, const uint16_t* q,
                                 const uint16_t* k, float* acc0, void* ws, hipStream_t stream) {
  float2* stat = static_cast<float2*>(ws);
  const int nb = (T + kPsBlockRows - 1) / kPsBlockRows;
  const int nh = batch * hq, ng = batch * hkv;
  const dim3 g1(static_cast<unsigned>(nh) * nb), g2(static_cast<unsigned>(ng) * nb);
  if (d == 128) {
    ps_rowstat_kernel<128><<<g1, kPsThreads, 0, stream>>>(q, k, hq, hkv, T, nh, nb, stat);
    ps_colsum_kernel<128><<<g2, kPsThreads, 0, stream>>>(q, k, hq, hkv, T, ng, stat, acc0);
  } else if (d == 64) {
    ps_rowstat_kernel<64><<<g1, kPsThreads, 0, stream>>>(q, k, hq, hkv, T, nh, nb, stat);
    ps_colsum_kernel<64><<<g2, kPsThreads, 0, stream>>>(q, k, hq, hkv, T, ng, stat, acc0);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mikv
