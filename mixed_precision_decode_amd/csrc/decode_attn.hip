// Mixed-precision decode attention over the two-tier MiKV cache.
//
// velog notes "No Token Left Behind ...", section 3.4 and paperlayer summary
// of arXiv 2402.18096, section 3.4: decode attention is a memory-bound
// batched matrix-vector product; keys/values are stored at low precision in
// precision-grouped tiers (allowed by the permutation invariance of
// attention) while the query and the attention map stay floating point.
// velog notes, Key contributions 2): q-hat = q / b pairs with the balanced
// keys k * b.
//
// Split-K ("flash-decoding") in two launches:
//   split kernel  one block per (sequence, kv head, query-head tile, split);
//                 a split is a slot range of ONE tier. Every thread first
//                 issues all of its key and value loads (TPT tokens), then
//                 computes scores (kept in registers), the split maximum,
//                 p = exp2(s - max) and sum p*v. Rows are streamed once:
//                   FP16 tier: d/8 lanes per token, 16-byte fp16 loads;
//                   low-bit tier: LPTQ lanes per token, packed-code loads,
//                   score = scale*sum(q*code) + zero*sum(q) per group,
//                   o += (p*scale)*code + p*zero per group.
//                 The block owning FP16 slot free16 appends the new token.
//   merge kernel  one block per (sequence, kv head): combines the split
//                 partials (max, sum, o) of every query head of the group and
//                 turns the FP16-tier scores into p16 (summed over the group).
// Scores are kept in the log2 domain (q-hat is pre-multiplied by
// log2(e)/sqrt(d)).
#include "common.hpp"
#include "kernels.hpp"

namespace mikv {

constexpr int kThreads = 256;
#ifndef MIKV_TPT
#define MIKV_TPT 8
#endif
constexpr int kTPT = MIKV_TPT;  // tokens per thread in a split
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeK {
  int hq, hkv, rep, cap16, capq, nq, len, group;
  int S16, Sq, C16, Cq, tiles;
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const float* b;
  uint16_t* k16;
  uint16_t* v16;
  int32_t* pos16;
  const int32_t* free16;
  const uint8_t* kq;
  const uint8_t* vq;
  const uint32_t* ksz;
  const uint32_t* vsz;
  float* o;
  float* p16;
  float2* part_ml;  // [units][tiles][S][RT]  (max, sum) per split and head
  float* part_o;    // [units][tiles][S][RT][D]
  float* sc16;      // [units][rep][cap16] scores of the FP16 tier
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int BITS, int CPL>
__device__ __forceinline__ void unpack_codes(const uint32_t* w, float (&c)[CPL]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int i = 0; i < CPL / 8; ++i) {
      const uint32_t lo = w[i] & 0x0F0F0F0Fu;
      const uint32_t hi = (w[i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c[8 * i + 2 * k] = static_cast<float>((lo >> (8 * k)) & 0xFFu);
        c[8 * i + 2 * k + 1] = static_cast<float>((hi >> (8 * k)) & 0xFFu);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < CPL / 16; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t m = (w[i] >> (2 * j)) & 0x03030303u;
#pragma unroll
        for (int k = 0; k < 4; ++k) c[16 * i + 4 * k + j] = static_cast<float>((m >> (8 * k)) & 0xFFu);
      }
    }
  }
}

template <int NW>
struct Words { uint32_t w[NW]; };

template <int NW>
__device__ __forceinline__ Words<NW> load_words(const uint8_t* p) {
  Words<NW> r;
  if constexpr (NW == 4) {
    const uint4 t = *reinterpret_cast<const uint4*>(p);
    r.w[0] = t.x; r.w[1] = t.y; r.w[2] = t.z; r.w[3] = t.w;
  } else if constexpr (NW == 2) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    r.w[0] = t.x; r.w[1] = t.y;
  } else {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
  return r;
}

// Sum over lanes sharing (lane % LPT) across the whole wave.
template <int LPT>
__device__ __forceinline__ float fold_slots(float v) {
  if constexpr (LPT <= 1) v += dpp<0x121>(v);
  if constexpr (LPT <= 2) v += dpp<0x122>(v);
  if constexpr (LPT <= 4) v += dpp<0x124>(v);
  if constexpr (LPT <= 8) v += dpp<0x128>(v);
  v += shfl_xor_f(v, 16);
  v += shfl_xor_f(v, 32);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}

// Block-wide: per-head maximum of the per-thread maxima (4 waves).
template <int RT>
__device__ __forceinline__ void block_max(float (&m)[RT], float (*sm)[RT], float* out) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const float w = wave_max(m[r]);
    if (lane == 0) sm[wave][r] = w;
  }
  __syncthreads();
  if (threadIdx.x < RT) {
    const int r = threadIdx.x;
    out[r] = fmaxf(fmaxf(sm[0][r], sm[1][r]), fmaxf(sm[2][r], sm[3][r]));
  }
  __syncthreads();
}

// Write the split partial: per-thread acc[RT][CPL] over channel slice
// c0 = lane*CPL (lane = tid % LPT) and per-thread lsum[RT].
template <int D, int RT, int LPT, int CPL>
__device__ __forceinline__ void write_partial(float (&acc)[RT][CPL], float (&lsum)[RT], const float* M,
                                              float* red, float* po, float2* pml) {
  const int tid = threadIdx.x, wave = tid / kWave, lane64 = tid % kWave;
  const int lane = tid % LPT;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[r][i] = fold_slots<LPT>(acc[r][i]);
    lsum[r] = fold_slots<LPT>(lsum[r]);
  }
  if (lane64 < LPT) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) red[(wave * RT + r) * D + lane * CPL + i] = acc[r][i];
    }
    if (lane64 == 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r) red[4 * RT * D + wave * RT + r] = lsum[r];
    }
  }
  __syncthreads();
  for (int i = tid; i < RT * D; i += kThreads) {
    const int r = i / D;
    po[i] = red[(0 * RT + r) * D + i % D] + red[(1 * RT + r) * D + i % D] +
            red[(2 * RT + r) * D + i % D] + red[(3 * RT + r) * D + i % D];
  }
  if (tid < RT) {
    const float* l = red + 4 * RT * D;
    pml[tid] = make_float2(M[tid], l[tid] + l[RT + tid] + l[2 * RT + tid] + l[3 * RT + tid]);
  }
}

template <int D, int BITS, int RT, int LPTQ>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(const DecodeK p) {
  const int S = p.S16 + p.Sq;
  const int split = blockIdx.x % S;
  const int rest = blockIdx.x / S;
  const int tile = rest % p.tiles;
  const int unit = rest / p.tiles;
  const int n = unit / p.hkv;
  const int g = unit % p.hkv;
  const int tid = threadIdx.x;
  const float qscale = kLog2e / sqrtf(static_cast<float>(D));
  const float* bvec = p.b + static_cast<int64_t>(unit) * D;
  const int part = (unit * p.tiles + tile) * S + split;
  float* po = p.part_o + static_cast<int64_t>(part) * RT * D;
  float2* pml = p.part_ml + static_cast<int64_t>(part) * RT;

  __shared__ float red[4 * RT * D + 4 * RT];
  __shared__ float sm_max[4][RT];
  __shared__ float sm_M[RT];

  if (split < p.S16) {
    // ---------------- FP16 tier ----------------
    constexpr int LPT = D / 8, CPL = 8, SLOTS = kThreads / LPT;
    const int lane = tid % LPT, tslot = tid / LPT, c0 = lane * CPL;
    const int s0 = split * p.C16;
    const int s1 = min(p.cap16, s0 + p.C16);
    const int fr = p.free16[unit];
    const int64_t rb = static_cast<int64_t>(unit) * p.cap16;
    uint4 kr[kTPT] = {}, vr[kTPT] = {};
#pragma unroll
    for (int j = 0; j < kTPT; ++j) {
      const int t = s0 + j * SLOTS + tslot;
      if (t < s1) {
        kr[j] = *reinterpret_cast<const uint4*>(p.k16 + (rb + t) * D + c0);
        vr[j] = *reinterpret_cast<const uint4*>(p.v16 + (rb + t) * D + c0);
      }
    }
    float qh[RT][CPL];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int h = g * p.rep + tile * RT + r;
      float qv[8];
      load8(p.q + (static_cast<int64_t>(n) * p.hq + h) * D + c0, qv);
#pragma unroll
      for (int i = 0; i < CPL; ++i) qh[r][i] = qv[i] * __builtin_amdgcn_rcpf(bvec[c0 + i]) * qscale;
    }
    // the new token replaces the free slot's stale row (and is appended)
    if (fr >= s0 && fr < s1 && (fr - s0) % SLOTS == tslot) {
      const int j = (fr - s0) / SLOTS;
      const int64_t nb = static_cast<int64_t>(unit) * D + c0;
      float kn[8];
      load8(p.k_new + nb, kn);
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = f2h(mul_rn(kn[2 * i], bvec[c0 + 2 * i]));
        const uint32_t hi = f2h(mul_rn(kn[2 * i + 1], bvec[c0 + 2 * i + 1]));
        w[i] = lo | (hi << 16);
      }
      const uint4 kv = make_uint4(w[0], w[1], w[2], w[3]);
      const uint4 vv = *reinterpret_cast<const uint4*>(p.v_new + nb);
#pragma unroll
      for (int jj = 0; jj < kTPT; ++jj)
        if (jj == j) { kr[jj] = kv; vr[jj] = vv; }
      if (tile == 0) {
        *reinterpret_cast<uint4*>(p.k16 + (rb + fr) * D + c0) = kv;
        *reinterpret_cast<uint4*>(p.v16 + (rb + fr) * D + c0) = vv;
        if (lane == 0) p.pos16[rb + fr] = p.len - 1;
      }
    }
    float sc[kTPT][RT];
    float mloc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) mloc[r] = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTPT; ++j) {
      const int t = s0 + j * SLOTS + tslot;
      const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kr[j]);
      float kx[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) { kx[2 * i] = lo_h(kw[i]); kx[2 * i + 1] = hi_h(kw[i]); }
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        float dot = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) dot += qh[r][i] * kx[i];
        dot = group_sum<LPT>(dot);
        sc[j][r] = (t < s1) ? dot : -INFINITY;
        mloc[r] = fmaxf(mloc[r], sc[j][r]);
        if (lane == 0 && t < s1)
          p.sc16[(static_cast<int64_t>(unit) * p.rep + tile * RT + r) * p.cap16 + t] = dot;
      }
    }
    block_max<RT>(mloc, sm_max, sm_M);
    float acc[RT][CPL], lsum[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      lsum[r] = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[r][i] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kTPT; ++j) {
      const int t = s0 + j * SLOTS + tslot;
      if (t < s1) {
        const uint32_t* vw = reinterpret_cast<const uint32_t*>(&vr[j]);
        float vx[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) { vx[2 * i] = lo_h(vw[i]); vx[2 * i + 1] = hi_h(vw[i]); }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const float pr = fast_exp2(sc[j][r] - sm_M[r]);
          lsum[r] += pr;
#pragma unroll
          for (int i = 0; i < CPL; ++i) acc[r][i] += pr * vx[i];
        }
      }
    }
    write_partial<D, RT, LPT, CPL>(acc, lsum, sm_M, red, po, pml);
  } else {
    // ---------------- low-bit tier ----------------
    constexpr int LPT = LPTQ, CPL = D / LPTQ, SLOTS = kThreads / LPT;
    constexpr int NB = CPL * BITS / 8, NW = NB / 4;
    constexpr int CB = D * BITS / 8;
    const int lane = tid % LPT, tslot = tid / LPT, c0 = lane * CPL;
    const int gpt = D / p.group;
    const int gi = c0 / p.group;
    const int t0 = (split - p.S16) * p.Cq;
    const int t1 = min(p.nq, t0 + p.Cq);
    const int64_t rb = static_cast<int64_t>(unit) * p.capq;
    Words<NW> kc[kTPT] = {}, vc[kTPT] = {};
    uint32_t ks[kTPT] = {}, vs[kTPT] = {};
#pragma unroll
    for (int j = 0; j < kTPT; ++j) {
      const int t = t0 + j * SLOTS + tslot;
      if (t < t1) {
        kc[j] = load_words<NW>(p.kq + (rb + t) * CB + lane * NB);
        ks[j] = p.ksz[(rb + t) * gpt + gi];
        vc[j] = load_words<NW>(p.vq + (rb + t) * CB + lane * NB);
        vs[j] = p.vsz[(rb + t) * gpt + gi];
      }
    }
    float sc[kTPT][RT];
    float mloc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) mloc[r] = -INFINITY;
    {
      float qh[RT][CPL], qsum[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int h = g * p.rep + tile * RT + r;
        const uint16_t* qp = p.q + (static_cast<int64_t>(n) * p.hq + h) * D + c0;
        qsum[r] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; i += 8) {
          float qv[8];
          load8(qp + i, qv);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            qh[r][i + e] = qv[e] * __builtin_amdgcn_rcpf(bvec[c0 + i + e]) * qscale;
            qsum[r] += qh[r][i + e];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kTPT; ++j) {
        const int t = t0 + j * SLOTS + tslot;
        float cf[CPL];
        unpack_codes<BITS, CPL>(kc[j].w, cf);
        const float s = lo_h(ks[j]), z = hi_h(ks[j]);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          float dot = 0.0f;
#pragma unroll
          for (int i = 0; i < CPL; ++i) dot += qh[r][i] * cf[i];
          float v = s * dot + z * qsum[r];
          v = group_sum<LPT>(v);
          sc[j][r] = (t < t1) ? v : -INFINITY;
          mloc[r] = fmaxf(mloc[r], sc[j][r]);
        }
      }
    }
    block_max<RT>(mloc, sm_max, sm_M);
    float acc[RT][CPL], lsum[RT], accz[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      lsum[r] = 0.0f;
      accz[r] = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[r][i] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kTPT; ++j) {
      const int t = t0 + j * SLOTS + tslot;
      if (t < t1) {
        float cf[CPL];
        unpack_codes<BITS, CPL>(vc[j].w, cf);
        const float s = lo_h(vs[j]), z = hi_h(vs[j]);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const float pr = fast_exp2(sc[j][r] - sm_M[r]);
          lsum[r] += pr;
          const float w = pr * s;
          accz[r] += pr * z;
#pragma unroll
          for (int i = 0; i < CPL; ++i) acc[r][i] += w * cf[i];
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[r][i] += accz[r];
    write_partial<D, RT, LPT, CPL>(acc, lsum, sm_M, red, po, pml);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(const DecodeK p, int RT) {
  extern __shared__ float sML[];  // [rep][2]
  const int unit = blockIdx.x;
  const int n = unit / p.hkv, g = unit % p.hkv;
  const int tid = threadIdx.x;
  const int S = p.S16 + p.Sq;
  for (int hl = tid; hl < p.rep; hl += kThreads) {
    const int tl = hl / RT, r = hl % RT;
    const float2* ml = p.part_ml + static_cast<int64_t>((unit * p.tiles + tl) * S) * RT + r;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[s * RT].x);
    float L = 0.0f;
    for (int s = 0; s < S; ++s) L += ml[s * RT].y * fast_exp2(ml[s * RT].x - M);
    sML[2 * hl] = M;
    sML[2 * hl + 1] = 1.0f / L;
  }
  __syncthreads();
  for (int i = tid; i < p.rep * D; i += kThreads) {
    const int hl = i / D, c = i % D;
    const int tl = hl / RT, r = hl % RT;
    const int64_t pb = static_cast<int64_t>((unit * p.tiles + tl) * S);
    const float M = sML[2 * hl];
    float v = 0.0f;
    for (int s = 0; s < S; ++s) {
      const float2 ml = p.part_ml[(pb + s) * RT + r];
      v += p.part_o[((pb + s) * RT + r) * D + c] * fast_exp2(ml.x - M);
    }
    p.o[(static_cast<int64_t>(n) * p.hq + g * p.rep + hl) * D + c] = v * sML[2 * hl + 1];
  }
  for (int sl = tid; sl < p.cap16; sl += kThreads) {
    float a = 0.0f;
    for (int hl = 0; hl < p.rep; ++hl) {
      const float s = p.sc16[(static_cast<int64_t>(unit) * p.rep + hl) * p.cap16 + sl];
      a += fast_exp2(s - sML[2 * hl]) * sML[2 * hl + 1];
    }
    p.p16[static_cast<int64_t>(unit) * p.cap16 + sl] = a;
  }
}

static inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// lanes per low-bit token: 4 for a single head (32 channels per lane at
// d = 128), 8 for head tiles (fewer registers per lane), never below 4 bytes
// of codes per lane
constexpr int lptq_for(int d, int bits, int RT) {
  return (RT == 1) ? 4 : ((d * bits / 32) < 8 ? (d * bits / 32) : 8);
}

DecodePlan decode_plan(int d, int bits, int rep, int cap16, int nq) {
  DecodePlan pl;
  pl.RT = (rep % 4 == 0) ? 4 : (rep % 2 == 0 ? 2 : 1);
  pl.tiles = rep / pl.RT;
  pl.C16 = (kThreads / (d / 8)) * kTPT;
  pl.Cq = (kThreads / lptq_for(d, bits, pl.RT)) * kTPT;
  pl.S16 = cdiv(cap16, pl.C16);
  pl.Sq = nq > 0 ? cdiv(nq, pl.Cq) : 0;
  return pl;
}

static inline size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t decode_ws_bytes(int batch, int hq, int hkv, int d, int cap16, const DecodePlan& pl) {
  const size_t units = static_cast<size_t>(batch) * hkv;
  const size_t rep = hq / hkv;
  const size_t nparts = units * pl.tiles * (pl.S16 + pl.Sq);
  return al256(nparts * pl.RT * sizeof(float2)) + al256(nparts * pl.RT * d * sizeof(float)) +
         al256(units * rep * cap16 * sizeof(float));
}

template <int D, int BITS, int RT>
static hipError_t launch_da(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
  DecodeK k;
  k.hq = a.hq; k.hkv = a.hkv; k.rep = a.hq / a.hkv; k.cap16 = a.cap16; k.capq = a.capq;
  k.nq = a.len - a.cap16; k.len = a.len; k.group = a.group;
  k.S16 = pl.S16; k.Sq = pl.Sq; k.C16 = pl.C16; k.Cq = pl.Cq; k.tiles = pl.tiles;
  k.q = a.q; k.k_new = a.k_new; k.v_new = a.v_new; k.b = a.b;
  k.k16 = a.k16; k.v16 = a.v16; k.pos16 = a.pos16; k.free16 = a.free16;
  k.kq = a.kq; k.vq = a.vq;
  k.ksz = reinterpret_cast<const uint32_t*>(a.ksz);
  k.vsz = reinterpret_cast<const uint32_t*>(a.vsz);
  k.o = a.o; k.p16 = a.p16;
  const size_t units = static_cast<size_t>(a.batch) * a.hkv;
  const size_t nparts = units * pl.tiles * (pl.S16 + pl.Sq);
  char* w = static_cast<char*>(a.ws);
  k.part_ml = reinterpret_cast<float2*>(w);
  w += al256(nparts * pl.RT * sizeof(float2));
  k.part_o = reinterpret_cast<float*>(w);
  w += al256(nparts * pl.RT * D * sizeof(float));
  k.sc16 = reinterpret_cast<float*>(w);
  constexpr int LPTQ = lptq_for(D, BITS, RT);
  decode_split_kernel<D, BITS, RT, LPTQ><<<static_cast<unsigned>(nparts), kThreads, 0, stream>>>(k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_merge_kernel<D><<<static_cast<unsigned>(units), kThreads, 2 * k.rep * sizeof(float), stream>>>(k, RT);
  return hipGetLastError();
}

hipError_t launch_decode_attn(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
#define MIKV_DA(D_, B_, RT_) \
  if (a.d == D_ && a.bits == B_ && pl.RT == RT_) return launch_da<D_, B_, RT_>(a, pl, stream);
  MIKV_DA(128, 4, 1) MIKV_DA(128, 4, 2) MIKV_DA(128, 4, 4)
  MIKV_DA(128, 2, 1) MIKV_DA(128, 2, 2) MIKV_DA(128, 2, 4)
  MIKV_DA(64, 4, 1) MIKV_DA(64, 4, 2) MIKV_DA(64, 4, 4)
  MIKV_DA(64, 2, 1) MIKV_DA(64, 2, 2) MIKV_DA(64, 2, 4)
#undef MIKV_DA
  return hipErrorInvalidValue;
}

}  // namespace mikv
