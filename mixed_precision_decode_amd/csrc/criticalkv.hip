// CriticalKV two-stage selection (gist.science summary of arXiv 2502.03805,
// "Algorithm 1": stage 1 takes alpha*budget entries with the largest
// attention weight; stage 2 takes the rest by attention weight times the L1
// norm of the value state projected by the output matrix W_O, the quantity
// the perturbation bound of the theoretical framework depends on).
//
// Kernels (one launch each, all on the caller's stream):
//   stage1  per head: radix top-b1 of A; marks stage-1 entries, writes -1 to
//           their score2 and the ascending list of the other rows.
//   wt      W_O rearranged per head as [hidden][d] (d contiguous), so that
//           every MFMA B operand is a run of 8 consecutive k.
//   project MFMA GEMM (v_mfma_f32_32x32x16_f16, fp32 accumulation) of the
//           listed V rows with the head's W_O slice, with the |.| row sum
//           fused into the epilogue so the [rows x hidden] product is never
//           stored: score2[i] = A[i] * sum_j |(V_i W_O,h)_j|.
//   stage2  per head: radix top-b2 of score2 outside stage 1, then the
//           ascending union of both stages.
// The projection is the only dense contraction of the method; it is the
// kernel bound by the matrix cores.
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace mikv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kCkvD = 128;     // head dim (contraction length)
constexpr int kBM = 256;       // rows per block (4 waves x 64)
constexpr int kBN = 64;        // hidden columns per step
constexpr int kLdw = kCkvD + 8;  // padded LDS row (halves) of the transposed W tile

struct CkvWs {
  uint8_t* s1;      // [H][T] stage-1 membership
  int32_t* rows2;   // [H][T - b1] rows outside stage 1, ascending
  float* score2;    // [H][T] used when the caller passes no score2
  uint16_t* wt;     // [H][hidden][d] W_O,h with the head dim contiguous
};

static inline size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

static CkvWs carve(void* ws, int H, int T) {
  char* w = static_cast<char*>(ws);
  CkvWs r;
  r.s1 = reinterpret_cast<uint8_t*>(w);
  w += al256(static_cast<size_t>(H) * T);
  r.rows2 = reinterpret_cast<int32_t*>(w);
  w += al256(static_cast<size_t>(H) * T * sizeof(int32_t));
  r.score2 = reinterpret_cast<float*>(w);
  w += al256(static_cast<size_t>(H) * T * sizeof(float));
  r.wt = reinterpret_cast<uint16_t*>(w);
  return r;
}

size_t criticalkv_ws_bytes(int H, int T, int d, int hidden) {
  return al256(static_cast<size_t>(H) * T) + al256(static_cast<size_t>(H) * T * sizeof(int32_t)) +
         al256(static_cast<size_t>(H) * T * sizeof(float)) +
         al256(static_cast<size_t>(H) * d * hidden * sizeof(uint16_t));
}

// ------------------------------------------------------------------ stage 1
// Stage kernels: one block of kStageThreads per head. After the radix
// select, positions are visited in chunks of kStageThreads * kRun; each thread
// takes kRun consecutive positions, so a chunk needs two block scans (ties,
// then the kept or rest positions) instead of two per kStageThreads positions.
constexpr int kStageThreads = 1024;
constexpr int kRun = 8;

__global__ __launch_bounds__(kStageThreads) void ckv_stage1_kernel(const float* __restrict__ A, int T, int b1,
                                                                   CkvWs w, float* __restrict__ score2) {
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const float* a = A + static_cast<int64_t>(h) * T;
  uint32_t tau = 0xFFFFFFFFu;
  int need = 0;
  if (b1 > 0) {
    block_radix_topm<kStageThreads, 32>(T, b1, [&](int i, uint32_t* key) {
      *key = float_key(a[i]);
      return true;
    }, &tau, &need);
  }
  int eq_seen = 0, nrest = 0;
  uint8_t* s1 = w.s1 + static_cast<int64_t>(h) * T;
  int32_t* rows2 = w.rows2 + static_cast<int64_t>(h) * (T - b1);
  float* sc = score2 + static_cast<int64_t>(h) * T;
  for (int p0 = 0; p0 < T; p0 += kStageThreads * kRun) {
    const int base = p0 + tid * kRun;
    uint32_t key[kRun];
    int neq = 0;
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      key[j] = (base + j < T) ? float_key(a[base + j]) : 0u;
      neq += (b1 > 0 && base + j < T && key[j] == tau) ? 1 : 0;
    }
    int eq_tot;
    int eq_rank = eq_seen + block_scan_add<kStageThreads>(neq, &eq_tot);
    eq_seen += eq_tot;
    bool sel[kRun];
    int nr = 0;
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      const bool valid = base + j < T;
      const bool eq = b1 > 0 && valid && key[j] == tau;
      sel[j] = valid && b1 > 0 && (key[j] > tau || (eq && eq_rank < need));
      eq_rank += eq ? 1 : 0;
      nr += (valid && !sel[j]) ? 1 : 0;
    }
    int r_tot;
    int rrank = nrest + block_scan_add<kStageThreads>(nr, &r_tot);
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      const int p = base + j;
      if (p < T) {
        s1[p] = sel[j] ? 1 : 0;
        if (sel[j]) sc[p] = -1.0f;
        else {
          if (rrank < T - b1) rows2[rrank] = p;
          ++rrank;
        }
      }
    }
    nrest += r_tot;
  }
}

// ------------------------------------------------------------------ W_O layout
// wt[h][n][k] = W_O[h*d + k][n]: one block per (64 columns, head) through an
// LDS tile [n][k] (row pitch kLdw halves, 16-byte aligned rows).
__global__ __launch_bounds__(256) void ckv_wt_kernel(const uint16_t* __restrict__ W, int hidden,
                                                     uint16_t* __restrict__ wt) {
  __shared__ __attribute__((aligned(16))) uint16_t t[kBN * kLdw];
  const int h = blockIdx.y, nb = blockIdx.x * kBN;
  const int tid = threadIdx.x;
  const uint16_t* src = W + static_cast<int64_t>(h) * kCkvD * hidden + nb;
#pragma unroll
  for (int i = 0; i < kCkvD * kBN / (8 * 256); ++i) {
    const int idx = tid + i * 256;
    const int k = idx / (kBN / 8), c = (idx % (kBN / 8)) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(k) * hidden + c);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      t[(c + j) * kLdw + k] = static_cast<uint16_t>((j & 1) ? (w4[j / 2] >> 16) : (w4[j / 2] & 0xFFFFu));
  }
  __syncthreads();
  uint16_t* dst = wt + (static_cast<int64_t>(h) * hidden + nb) * kCkvD;
#pragma unroll
  for (int i = 0; i < kCkvD * kBN / (8 * 256); ++i) {
    const int idx = tid + i * 256;
    const int n = idx / (kCkvD / 8), kc = (idx % (kCkvD / 8)) * 8;
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(n) * kCkvD + kc) =
        *reinterpret_cast<const uint4*>(&t[n * kLdw + kc]);
  }
}

// ------------------------------------------------------------------ projection
// Block: 256 threads = 4 waves; rows [blk*256, blk*256+256) of the head's
// row list; wave w owns 64 rows = two 32-row MFMA tiles. Hidden columns are
// walked in steps of 64: the wt tile [64 n][128 k] (16 KB, contiguous) is
// copied into one of two LDS buffers while the other one feeds the MFMAs, so
// each step needs a single barrier; every MFMA B operand is one 16-byte LDS
// read.
// MFMA 32x32x16 operand layout (lane l): A[l%32][8*(l/32) + 0..7],
// B[8*(l/32) + 0..7][l%32], D register r: row 8*(r/4) + 4*(l/32) + r%4,
// column l%32.
__global__ __launch_bounds__(256) void ckv_project_kernel(const float* __restrict__ A,
                                                              const uint16_t* __restrict__ V, int H,
                                                              int T, int hidden, int nrows, int mt,
                                                              CkvWs w, float* __restrict__ score2) {
  __shared__ __attribute__((aligned(16))) uint16_t wbuf[2][kBN * kLdw];
  int head, tile;
  if (H % 8 == 0) {
    // keep every block of a head on one XCD (blocks go round-robin over 8)
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
    head = xcd + 8 * (local / mt);
    tile = local % mt;
  } else {
    head = blockIdx.x / mt;
    tile = blockIdx.x % mt;
  }
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int32_t* rows2 = w.rows2 + static_cast<int64_t>(head) * nrows;
  const uint16_t* Vh = V + static_cast<int64_t>(head) * T * kCkvD;
  const uint16_t* Wh = w.wt + static_cast<int64_t>(head) * hidden * kCkvD;

  // wt tile copy: thread covers row n = tid / 4, k = 32 * (tid % 4) .. +31
  const int ln = tid / 4, lk = (tid % 4) * 32;
  uint4 w0, w1, w2, w3;
  auto load_w = [&](int nb) {
    const uint4* src = reinterpret_cast<const uint4*>(Wh + static_cast<int64_t>(nb + ln) * kCkvD + lk);
    w0 = src[0];
    w1 = src[1];
    w2 = src[2];
    w3 = src[3];
  };
  auto store_w = [&](int buf) {
    uint4* dst = reinterpret_cast<uint4*>(&wbuf[buf][ln * kLdw + lk]);
    dst[0] = w0;
    dst[1] = w1;
    dst[2] = w2;
    dst[3] = w3;
  };
  const int nsteps = hidden / kBN;
  load_w(0);

  // A operands: two 32-row tiles x 8 k-steps, held for the whole kernel
  half8 afrag[2][8];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int j = tile * kBM + wave * 64 + mi * 32 + lane % 32;
    const bool ok = j < nrows;
    const int src = ok ? min(max(rows2[j], 0), T - 1) : 0;  // clamp: rows2 comes from stage 1
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ok) {
        const uint4 t = *reinterpret_cast<const uint4*>(Vh + static_cast<int64_t>(src) * kCkvD + ks * 16 + (lane / 32) * 8);
        afrag[mi][ks] = __builtin_bit_cast(half8, t);
      } else {
        afrag[mi][ks] = half8{};
      }
    }
  }
  float rsum[2][16];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) rsum[mi][r] = 0.0f;

  store_w(0);
  if (nsteps > 1) load_w(kBN);
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const uint16_t* wt = wbuf[step & 1];
    // the MFMA phase runs at raised wave priority: the SIMD's arbiter issues
    // it ahead of the other resident wave's epilogue and tile copy
    __builtin_amdgcn_s_setprio(1);
    // four independent accumulator chains: 2 row tiles x 2 column tiles
    floatx16 c00 = {}, c10 = {}, c01 = {}, c11 = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int kofs = ks * 16 + (lane / 32) * 8;
      const half8 b0 = *reinterpret_cast<const half8*>(&wt[(lane % 32) * kLdw + kofs]);
      const half8 b1 = *reinterpret_cast<const half8*>(&wt[(32 + lane % 32) * kLdw + kofs]);
      c00 = __builtin_amdgcn_mfma_f32_32x32x16_f16(afrag[0][ks], b0, c00, 0, 0, 0);
      c10 = __builtin_amdgcn_mfma_f32_32x32x16_f16(afrag[1][ks], b0, c10, 0, 0, 0);
      c01 = __builtin_amdgcn_mfma_f32_32x32x16_f16(afrag[0][ks], b1, c01, 0, 0, 0);
      c11 = __builtin_amdgcn_mfma_f32_32x32x16_f16(afrag[1][ks], b1, c11, 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      rsum[0][r] += fabsf(c00[r]) + fabsf(c01[r]);
      rsum[1][r] += fabsf(c10[r]) + fabsf(c11[r]);
    }
    // the next tile goes into the other buffer, which every wave finished
    // reading before the previous barrier
    if (step + 1 < nsteps) {
      store_w((step + 1) & 1);
      if (step + 2 < nsteps) load_w((step + 2) * kBN);
    }
    __syncthreads();
  }
  // reduce over the 32 columns held by lanes with equal lane/32
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = rsum[mi][r];
      v = group_sum<16>(v);  // DPP within the row
      const LanePair x = pair_xor16(f2u(v));  // rows 0+1 and 2+3
      v = u2f(x.a) + u2f(x.b);
      rsum[mi][r] = v;
    }
  if (lane % 32 == 0) {
    const float* a = A + static_cast<int64_t>(head) * T;
    float* sc = score2 + static_cast<int64_t>(head) * T;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row_in_tile = 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
        const int j = tile * kBM + wave * 64 + mi * 32 + row_in_tile;
        if (j < nrows) {
          const int i = rows2[j];
          if (i >= 0 && i < T) sc[i] = a[i] * rsum[mi][r];
        }
      }
  }
}

// ------------------------------------------------------------------ stage 2
__global__ __launch_bounds__(kStageThreads) void ckv_stage2_kernel(int T, int b1, int b2, CkvWs w,
                                                                   const float* __restrict__ score2,
                                                                   int32_t* __restrict__ idx) {
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const uint8_t* s1 = w.s1 + static_cast<int64_t>(h) * T;
  const float* sc = score2 + static_cast<int64_t>(h) * T;
  uint32_t tau = 0xFFFFFFFFu;
  int need = 0;
  if (b2 > 0) {
    block_radix_topm<kStageThreads, 32>(T, b2, [&](int i, uint32_t* key) {
      if (s1[i]) return false;
      *key = float_key(sc[i]);
      return true;
    }, &tau, &need);
  }
  int eq_seen = 0, nsel = 0;
  int32_t* out = idx + static_cast<int64_t>(h) * (b1 + b2);
  for (int p0 = 0; p0 < T; p0 += kStageThreads * kRun) {
    const int base = p0 + tid * kRun;
    uint32_t key[kRun];
    bool in1[kRun];
    int neq = 0;
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      const bool valid = base + j < T;
      in1[j] = valid && s1[base + j] != 0;
      key[j] = (valid && !in1[j]) ? float_key(sc[base + j]) : 0u;
      neq += (b2 > 0 && valid && !in1[j] && key[j] == tau) ? 1 : 0;
    }
    int eq_tot;
    int eq_rank = eq_seen + block_scan_add<kStageThreads>(neq, &eq_tot);
    eq_seen += eq_tot;
    bool sel[kRun];
    int ns = 0;
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      const bool valid = base + j < T;
      const bool eq = b2 > 0 && valid && !in1[j] && key[j] == tau;
      sel[j] = valid && (in1[j] || (b2 > 0 && (key[j] > tau || (eq && eq_rank < need))));
      eq_rank += eq ? 1 : 0;
      ns += sel[j] ? 1 : 0;
    }
    int s_tot;
    int rank = nsel + block_scan_add<kStageThreads>(ns, &s_tot);
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      if (sel[j]) {
        if (rank < b1 + b2) out[rank] = base + j;
        ++rank;
      }
    }
    nsel += s_tot;
  }
}

hipError_t launch_criticalkv(const float* A, const uint16_t* V, const uint16_t* W, int H, int T,
                             int d, int hidden, int b1, int b2, int32_t* idx, float* score2,
                             void* ws, hipStream_t stream) {
  if (d != kCkvD || hidden % kBN != 0) return hipErrorInvalidValue;
  CkvWs w = carve(ws, H, T);
  float* sc = score2 ? score2 : w.score2;
  ckv_stage1_kernel<<<H, kStageThreads, 0, stream>>>(A, T, b1, w, sc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nrows = T - b1;
  if (nrows > 0) {
    ckv_wt_kernel<<<dim3(hidden / kBN, H), 256, 0, stream>>>(W, hidden, w.wt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int mt = (nrows + kBM - 1) / kBM;
    ckv_project_kernel<<<H * mt, 256, 0, stream>>>(A, V, H, T, hidden, nrows, mt, w, sc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ckv_stage2_kernel<<<H, kStageThreads, 0, stream>>>(T, b1, b2, w, sc, idx);
  return hipGetLastError();
}

}  // namespace mikv
