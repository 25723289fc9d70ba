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
//   pass 1 (rowstat)  one wave per (sequence, query head, 64 queries); the
//                     queries' rows are the held B operand, the causal key
//                     tiles stream through the A operand; each lane keeps an
//                     online (max, sum) of its column; the two lanes of a
//                     column combine at the end -> lse_i = M_i + log2(L_i),
//                     the row's log-sum-exp in log2 units.
//   pass 2 (colsum)   one wave per (sequence, kv head, 64 keys); the keys'
//                     rows are the held A operand; every query tile at or
//                     after the diagonal of every head of the group streams
//                     through the B operand; p = exp2(s - lse_i) is summed
//                     per key row in registers, then across the 32 lanes
//                     that share the rows -> acc0.
// A wave holds two 32-row tiles, so every streamed tile feeds two
// independent MFMA chains.
// The two passes compute bit-identical scores (same operands, same MFMA
// sequence), so every p <= 1. Only the diagonal tile of a wave is masked.
// The streamed operand tile (keys in pass 1, queries in pass 2) is shared by
// the block's four waves through LDS. No atomics: each wave owns its
// outputs. Blocks with the most tiles are dispatched first.
#include <cfloat>

#include "common.hpp"
#include "kernels.hpp"

namespace mikv {

namespace {

typedef _Float16 ps_half8 __attribute__((ext_vector_type(8)));
typedef float ps_floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned ps_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPsWaves = 4;                 // waves per block
constexpr int kPsThreads = kPsWaves * kWave;
constexpr int kPsTile = 32;                 // rows of one MFMA operand tile
constexpr int kPsTilesPerWave = 2;          // operand tiles a wave holds
constexpr int kPsWaveRows = kPsTilesPerWave * kPsTile;
constexpr int kPsBlockRows = kPsWaves * kPsWaveRows;
constexpr float kPsLog2e = 1.4426950408889634f;
// Both kernels are compiled for at least three waves per SIMD (168 VGPRs):
// left to itself the compiler took 170-190 registers, two waves per SIMD,
// and the passes ran 15% slower.
constexpr int kPsMinWaves = 3;

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

// key row of accumulator register r within a 32-row tile
__device__ __forceinline__ int row_of(int r, int lane) { return 8 * (r / 4) + 4 * (lane / 32) + (r % 4); }

__device__ __forceinline__ float ps_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS staging of the streamed 32-row tile, shared by the block's four waves.
// The block copies a tile with coalesced 16-byte loads (consecutive threads,
// consecutive bytes of consecutive rows) into one of two buffers while the
// waves read MFMA operands from the other; rows are padded by 16 bytes so
// that the operand reads of the 32 rows spread over the LDS banks.
template <int D>
struct PsStage {
  static constexpr int kStride = D + 8;                  // halves per LDS row
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  static constexpr int kRowsPerPass = kPsThreads / kChunks;
  static constexpr int kPasses = kPsTile / kRowsPerPass;  // loads per thread and tile
  static_assert(kPasses == 1 || kPasses == 2, "a 32-row tile is one or two passes of the block");
  ps_u32x4 r0, r1;  // native vectors (HIP's uint4 struct here was left in scratch memory)
  // rows row0 .. row0 + 31 of base (clamped to the last row)
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int row0, int T) {
    const int tid = threadIdx.x;
    const uint16_t* p = base + 8 * (tid % kChunks);
    r0 = *reinterpret_cast<const ps_u32x4*>(p + static_cast<int64_t>(min(row0 + tid / kChunks, T - 1)) * D);
    if constexpr (kPasses == 2)
      r1 = *reinterpret_cast<const ps_u32x4*>(
          p + static_cast<int64_t>(min(row0 + kRowsPerPass + tid / kChunks, T - 1)) * D);
  }
  __device__ __forceinline__ void store(uint16_t* buf) const {
    const int tid = threadIdx.x;
    uint16_t* p = buf + (tid / kChunks) * kStride + 8 * (tid % kChunks);
    *reinterpret_cast<ps_u32x4*>(p) = r0;
    if constexpr (kPasses == 2) *reinterpret_cast<ps_u32x4*>(p + kRowsPerPass * kStride) = r1;
  }
  // the lane's MFMA operand slices of the staged tile (row l % 32)
  static __device__ __forceinline__ void operand(const uint16_t* buf, ps_half8 (&f)[D / 16]) {
    const int lane = threadIdx.x % kWave;
    const uint16_t* p = buf + (lane % 32) * kStride + 8 * (lane / 32);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) f[ks] = *reinterpret_cast<const ps_half8*>(p + 16 * ks);
  }
};

template <int D>
__global__ __launch_bounds__(kPsThreads, kPsMinWaves) void ps_rowstat_kernel(const uint16_t* __restrict__ q,
                                                                  const uint16_t* __restrict__ k, int hq,
                                                                  int hkv, int T, int nh, int nib,
                                                                  float* __restrict__ lse) {
  constexpr int KS = D / 16;
  using Stage = PsStage<D>;
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][kPsTile * Stage::kStride];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  // the last query blocks (most key tiles) first
  const int ib = nib - 1 - static_cast<int>(blockIdx.x) / nh;
  const int nhi = static_cast<int>(blockIdx.x) % nh;  // n * hq + h
  const int n = nhi / hq, h = nhi % hq;
  const int g = h / (hq / hkv);
  // the wave's queries: two tiles of 32, i0 .. i0 + 63
  const int i0 = ib * kPsBlockRows + wave * kPsWaveRows;
  const bool active = i0 < T;  // every wave takes part in the copies and barriers
  const uint16_t* kb = k + (static_cast<int64_t>(n) * hkv + g) * T * D;
  const uint16_t* qb = q + static_cast<int64_t>(nhi) * T * D;
  int iq[kPsTilesPerWave];
  ps_half8 bq[kPsTilesPerWave][KS];
#pragma unroll
  for (int u = 0; u < kPsTilesPerWave; ++u) {
    iq[u] = i0 + u * kPsTile + lane % 32;  // this lane's query column in tile u
    load_rows<D>(qb, min(iq[u], T - 1), bq[u]);
  }
  const float c = kPsLog2e / sqrtf(static_cast<float>(D));
  // key tiles 0 .. diag + u for query tile u (its diagonal tile holds t = i
  // and is the only one with keys after some of its queries); the block
  // walks the tiles of its last active wave
  const int diag = i0 / kPsTile;
  const int last = min(ib * kPsBlockRows + kPsBlockRows - 1, T - 1) / kPsTile;
  float m[kPsTilesPerWave], l[kPsTilesPerWave];  // log2-domain running max and sum per column
#pragma unroll
  for (int u = 0; u < kPsTilesPerWave; ++u) m[u] = -INFINITY, l[u] = 0.0f;
  Stage st;
  st.load(kb, 0, T);
  st.store(kt[0]);
  __syncthreads();
  for (int tt = 0; tt <= last; ++tt) {
    if (tt < last) st.load(kb, (tt + 1) * kPsTile, T);
    if (active && tt <= diag + kPsTilesPerWave - 1) {
      ps_half8 ka[KS];
      Stage::operand(kt[tt & 1], ka);
      ps_floatx16 s[kPsTilesPerWave];
      // independent accumulator chains for the query tiles
#pragma unroll
      for (int u = 0; u < kPsTilesPerWave; ++u) s[u] = ps_floatx16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int u = 0; u < kPsTilesPerWave; ++u)
          s[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[ks], bq[u][ks], s[u], 0, 0, 0);
      const int t0 = tt * kPsTile;
#pragma unroll
      for (int u = 0; u < kPsTilesPerWave; ++u) {
        if (tt > diag + u) continue;  // keys all after tile u's queries
        if (tt == diag + u) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (t0 + row_of(r, lane) > iq[u]) s[u][r] = -INFINITY;  // causal
        }
        float mx = s[u][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[u][r]);
        const float mn = fmaxf(m[u], mx * c);
        const float mref = fmaxf(mn, -FLT_MAX);  // exp2(-inf - mref) = 0 while nothing is seen
        float lu = l[u] * ps_exp2(m[u] - mref);
        m[u] = mn;
#pragma unroll
        for (int r = 0; r < 16; ++r) lu += ps_exp2(fmaf(s[u][r], c, -mref));
        l[u] = lu;
      }
    }
    // the other buffer was last read before the previous barrier
    if (tt < last) st.store(kt[(tt + 1) & 1]);
    __syncthreads();
  }
  if (!active) return;
#pragma unroll
  for (int u = 0; u < kPsTilesPerWave; ++u) {
    // lanes l and l + 32 hold the two halves of column i's key rows
    // (the pairs hold lanes l and l ^ 32 in the same order for m and l; the
    // combine is symmetric in the two)
    const LanePair pm = pair_xor32(f2u(m[u])), pl = pair_xor32(f2u(l[u]));
    const float ma = u2f(pm.a), mb = u2f(pm.b);
    const float M = fmaxf(ma, mb);  // finite: key t = i is in lane l or l + 32
    const float L = u2f(pl.a) * ps_exp2(ma - M) + u2f(pl.b) * ps_exp2(mb - M);  // >= 1
    // log2-sum-exp of the row: p[i][t] = exp2(s[i][t] * c - lse[i])
    if (lane < 32 && iq[u] < T) lse[static_cast<int64_t>(nhi) * T + iq[u]] = M + __builtin_amdgcn_logf(L);
  }
}

template <int D>
__global__ __launch_bounds__(kPsThreads, kPsMinWaves) void ps_colsum_kernel(const uint16_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ k, int hq,
                                                                 int hkv, int T, int ng,
                                                                 const float* __restrict__ lse,
                                                                 float* __restrict__ acc0) {
  constexpr int KS = D / 16;
  using Stage = PsStage<D>;
  __shared__ __attribute__((aligned(16))) uint16_t qt[2][kPsTile * Stage::kStride];
  __shared__ float qlse[2][kPsTile];
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  // the first key blocks (most query tiles) first
  const int tb = static_cast<int>(blockIdx.x) / ng;
  const int ngi = static_cast<int>(blockIdx.x) % ng;  // n * hkv + g
  const int n = ngi / hkv, g = ngi % hkv;
  const int rep = hq / hkv;
  // the wave's keys: two tiles of 32, t0 .. t0 + 63
  const int t0 = tb * kPsBlockRows + wave * kPsWaveRows;
  const bool active = t0 < T;  // every wave takes part in the copies and barriers
  ps_half8 ka[kPsTilesPerWave][KS];
#pragma unroll
  for (int u = 0; u < kPsTilesPerWave; ++u)
    load_rows<D>(k + static_cast<int64_t>(ngi) * T * D, min(t0 + u * kPsTile + lane % 32, T - 1), ka[u]);
  const float c = kPsLog2e / sqrtf(static_cast<float>(D));
  float col[kPsTilesPerWave][16];
#pragma unroll
  for (int u = 0; u < kPsTilesPerWave; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) col[u][r] = 0.0f;
  // the block walks query tiles first .. ntiles-1 of every head of the
  // group; key tile u of the wave starts at its diagonal query tile diag + u
  const int first = tb * (kPsBlockRows / kPsTile), ntiles = (T - 1) / kPsTile + 1;
  const int per_head = ntiles - first;
  const int total = rep * per_head;
  const int diag = t0 / kPsTile;
  Stage st;
  float ls = 0.0f;
  // iteration j: head g*rep + j / per_head, query tile first + j % per_head
  auto fetch = [&](int j) {
    const int nhi = n * hq + g * rep + j / per_head;
    const int i0 = (first + j % per_head) * kPsTile;
    st.load(q + static_cast<int64_t>(nhi) * T * D, i0, T);
    // a query past the prompt contributes nothing: exp2(-inf)
    if (tid < kPsTile) ls = (i0 + tid < T) ? lse[static_cast<int64_t>(nhi) * T + i0 + tid] : INFINITY;
  };
  auto stage = [&](int buf) {
    st.store(qt[buf]);
    if (tid < kPsTile) qlse[buf][tid] = ls;
  };
  fetch(0);
  stage(0);
  __syncthreads();
  for (int j = 0; j < total; ++j) {
    if (j + 1 < total) fetch(j + 1);
    const int it = first + j % per_head;
    if (active && it >= diag) {
      ps_half8 bq[KS];
      Stage::operand(qt[j & 1], bq);
      const float li = qlse[j & 1][lane % 32];
      const int i = it * kPsTile + lane % 32;
      ps_floatx16 s[kPsTilesPerWave];
#pragma unroll
      for (int u = 0; u < kPsTilesPerWave; ++u) s[u] = ps_floatx16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int u = 0; u < kPsTilesPerWave; ++u)
          s[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[u][ks], bq[ks], s[u], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < kPsTilesPerWave; ++u) {
        if (it < diag + u) continue;  // queries all before tile u's keys
        if (it == diag + u) {         // diagonal tile: causal mask
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (t0 + u * kPsTile + row_of(r, lane) > i) s[u][r] = -INFINITY;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) col[u][r] += ps_exp2(fmaf(s[u][r], c, -li));
      }
    }
    if (j + 1 < total) stage((j + 1) & 1);
    __syncthreads();
  }
  if (!active) return;
  // sum over the 32 query columns of the lanes that share l / 32
#pragma unroll
  for (int u = 0; u < kPsTilesPerWave; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = col[u][r];
      v = group_sum<16>(v);  // DPP within the row
      const LanePair x = pair_xor16(f2u(v));  // rows 0+1 and 2+3
      v = u2f(x.a) + u2f(x.b);
      col[u][r] = v;
    }
  if (lane % 32 == 0) {
    float* out = acc0 + static_cast<int64_t>(ngi) * T;
#pragma unroll
    for (int u = 0; u < kPsTilesPerWave; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + u * kPsTile + row_of(r, lane);
        if (t < T) out[t] = col[u][r];
      }
  }
}

}  // namespace

size_t prefill_scores_ws_bytes(int batch, int hq, int T) {
  return static_cast<size_t>(batch) * hq * T * sizeof(float);
}

hipError_t launch_prefill_scores(int batch, int hq, int hkv, int d, int T, const uint16_t* q,
                                 const uint16_t* k, float* acc0, void* ws, hipStream_t stream) {
  float* stat = static_cast<float*>(ws);
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
