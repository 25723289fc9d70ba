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
//                 a split is a contiguous slot range of ONE tier, sized so
//                 that every block streams about the same number of bytes.
//                 The block walks its range in batches; each thread keeps an
//                 online softmax (running max, sum, p*v) for its tokens and
//                 prefetches the next batch while it computes the current
//                 one, so loads stay in flight without block barriers.
//                   FP16 tier: d/8 lanes per token, 16-byte fp16 row loads.
//                   low-bit tier: LPTQ lanes per token, packed-code loads;
//                   score = scale*sum(q*code) + zero*sum(q) per group,
//                   o += (p*scale)*code + p*zero per group (rows are never
//                   widened in memory).
//                 The block owning FP16 slot free16 appends the new token.
//   merge kernel  one block per (sequence, kv head): combines the split
//                 partials of every query head of the group and turns the
//                 FP16-tier scores into p16 (summed over the group).
// Per-channel key tiles (velog notes, the per-channel alternative and its
// appendix C summary): the low-bit tier holds whole tiles of 64 tokens, each
// key channel with its own (scale, zero) per tile; a block first builds a
// table of q-hat * scale and sum(q-hat * zero) per tile and head in LDS, and
// a key score is then table . code + that sum. The fp16 buffer of pairs
// waiting for a tile is one more split, streamed like the FP16 tier.
// Tiles of 2-4 query heads with groups of d/2 channels run the split step as
// decode_tile_kernel (decode_tile.hpp): key scores on the matrix cores, one
// lane per (token, heads) for the softmax, value sums on the vector ALUs.
// Scores are in the log2 domain (q-hat is pre-multiplied by log2(e)/sqrt(d)).
#include <atomic>
#include <hip/hip_ext.h>
#include <cfloat>

#include "common.hpp"
#include "kernels.hpp"
#include "h2o_common.hpp"

namespace mikv {

constexpr int kThreads = 256;
#ifndef MIKV_TPT16
#define MIKV_TPT16 4
#endif
#ifndef MIKV_TPTQ
#define MIKV_TPTQ 2
#endif
#ifndef MIKV_BLOCKS_PER_CU
#define MIKV_BLOCKS_PER_CU 4
#endif
constexpr int kTPT16 = MIKV_TPT16;  // FP16 tokens per thread per batch
constexpr int kTPTQ = MIKV_TPTQ;    // low-bit tokens per thread per batch
constexpr float kLog2e = 1.4426950408889634f;


struct DecodeK {
  int hq, hkv, rep, cap16, capq, nq, len, group, units;
  int S16, Sq, C16, Cq, tiles, f16_first;
  int Sb, nb;         // per-channel key tiles: buffer splits (0 or 1) and buffered pairs
  const uint32_t* kcsz;  // [units][capq/64][D] (scale | zero << 16) per tile and channel
  const uint16_t* kbuf;  // [units][64][D] fp16 buffered pairs
  const uint16_t* vbuf;
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
  uint8_t* kimp;      // importance tier as codes (reduced-precision importance cache)
  uint8_t* vimp;
  uint32_t* kimpsz;
  uint32_t* vimpsz;
  float* o;
  float* p16;
  float2* part_ml;  // [units][tiles][S][RT]  (max, sum) per split and head
  float* part_o;    // [units][tiles][S][RT][D]
  float* sc16;      // [units][rep][cap16] scores of the FP16 tier
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The empty asm keeps the masked word opaque so that each byte converts with
// one v_cvt_f32_ubyteN instead of a bit-field extract plus a conversion.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int BITS, int CPL>
__device__ __forceinline__ void unpack_codes(const uint32_t* w, float (&c)[CPL]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int i = 0; i < CPL / 8; ++i) {
      const uint32_t lo = opaque(w[i] & 0x0F0F0F0Fu);
      const uint32_t hi = opaque((w[i] >> 4) & 0x0F0F0F0Fu);
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
        const uint32_t m = opaque((w[i] >> (2 * j)) & 0x03030303u);
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
    const uint4 t = ld_nt16(p);
    r.w[0] = t.x; r.w[1] = t.y; r.w[2] = t.z; r.w[3] = t.w;
  } else if constexpr (NW == 2) {
    const uint2 t = ld_nt8(p);
    r.w[0] = t.x; r.w[1] = t.y;
  } else {
    r.w[0] = ld_nt4(p);
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
  return rows_sum(v);
}

// Online-softmax state of one thread for RT heads and CPL channels.
template <int RT, int CPL>
struct Acc {
  float m[RT], l[RT], z[RT];
  float a[RT][CPL];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      m[r] = -INFINITY; l[r] = 0.0f; z[r] = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) a[r][i] = 0.0f;
    }
  }
  // raise the running max of head r to at least mb, rescaling the sums
  __device__ __forceinline__ void rebase(int r, float mb) {
    const float mn = fmaxf(m[r], mb);
    if (mn > m[r]) {
      const float f = fast_exp2(m[r] - mn);  // 0 when m was -inf
      l[r] *= f;
      z[r] *= f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) a[r][i] *= f;
      m[r] = mn;
    }
  }
};

// Combine the block's per-thread states into one partial (max, sum, o).
template <int D, int RT, int LPT, int CPL>
__device__ __forceinline__ void write_partial(Acc<RT, CPL>& s, float* red, float (*sm)[RT],
                                              float* sM, float* po, float2* pml) {
  const int tid = threadIdx.x, wave = tid / kWave, lane64 = tid % kWave;
  const int lane = tid % LPT;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const float w = wave_max(s.m[r]);
    if (lane64 == 0) sm[wave][r] = w;
  }
  __syncthreads();
  if (tid < RT) sM[tid] = fmaxf(fmaxf(sm[0][tid], sm[1][tid]), fmaxf(sm[2][tid], sm[3][tid]));
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const float f = (s.m[r] == -INFINITY) ? 0.0f : fast_exp2(s.m[r] - sM[r]);
#pragma unroll
    for (int i = 0; i < CPL; ++i) s.a[r][i] = fold_slots<LPT>((s.a[r][i] + s.z[r]) * f);
    s.l[r] = fold_slots<LPT>(s.l[r] * f);
  }
  if (lane64 < LPT) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int i = 0; i < CPL; ++i) red[(wave * RT + r) * D + lane * CPL + i] = s.a[r][i];
    if (lane64 == 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r) red[4 * RT * D + wave * RT + r] = s.l[r];
    }
  }
  __syncthreads();
  for (int i = tid; i < RT * D; i += kThreads) {
    const int r = i / D, c = i % D;
    po[i] = red[(0 * RT + r) * D + c] + red[(1 * RT + r) * D + c] + red[(2 * RT + r) * D + c] +
            red[(3 * RT + r) * D + c];
  }
  if (tid < RT) {
    const float* l = red + 4 * RT * D;
    pml[tid] = make_float2(sM[tid], l[tid] + l[RT + tid] + l[2 * RT + tid] + l[3 * RT + tid]);
  }
}

// q-hat for the lane's CPL channels of the block's RT heads: fp32(q) times
// the hardware reciprocal of b (v_rcp_f32, within 1 ulp of 1/b) times
// log2(e)/sqrt(d); q-hat only feeds scores, which are compared to a
// tolerance.
template <int D, int RT, int CPL>
__device__ __forceinline__ void load_qhat(const DecodeK& p, int n, int g, int tile, int c0,
                                          const float* bvec, float (&qh)[RT][CPL]) {
  const float qscale = kLog2e / sqrtf(static_cast<float>(D));
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int h = g * p.rep + tile * RT + r;
    const uint16_t* qp = p.q + (static_cast<int64_t>(n) * p.hq + h) * D + c0;
#pragma unroll
    for (int i = 0; i < CPL; i += 8) {
      float qv[8];
      load8(qp + i, qv);
#pragma unroll
      for (int e = 0; e < 8; ++e) qh[r][i + e] = qv[e] * __builtin_amdgcn_rcpf(bvec[c0 + i + e]) * qscale;
    }
  }
}

// ---------------------------------------------------------------------------
// Low-bit tier.
//
// Buffer loads through a per-block resource that spans exactly the block's
// token range [t0, t1): the lane offset of a token is a 32-bit byte offset
// from t0, so no 64-bit address arithmetic runs per load, and a load past t1
// returns zeros without touching memory (scale 0 and zero 0, so such a token
// adds nothing once its score is masked). The prefetch of the batch after the
// last one is therefore issued unconditionally, which keeps the loop free of
// branches around loads.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kBufNT = 2;  // cache policy bit: nontemporal
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  // dword 3 of a raw (stride 0) gfx9 buffer resource: 32-bit data format
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
template <int NW>
__device__ __forceinline__ Words<NW> bload(Rsrc r, uint32_t off) {
  Words<NW> o;
  if constexpr (NW == 4) {
    const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kBufNT);
    o.w[0] = t[0]; o.w[1] = t[1]; o.w[2] = t[2]; o.w[3] = t[3];
  } else if constexpr (NW == 2) {
    const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, kBufNT);
    o.w[0] = t[0]; o.w[1] = t[1];
  } else {
    o.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, kBufNT);
  }
  return o;
}
__device__ __forceinline__ uint32_t bload1(Rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, kBufNT);
}

// fp16 pairs (1024 + code_a, 1024 + code_b) from one word of packed codes:
// each code is isolated in a byte, and v_perm puts it under a 0x64 byte, the
// fp16 1024 + code exactly (with magic = 0 under a zero byte instead: the
// fp16 subnormal code * 2^-24, also exact). Pair k of the word's CPW channels covers:
//   INT4 (channels at bits 4c): k = 0,1 even channels (4k, 4k+2), k = 2,3 odd
//        channels (4(k-2)+1, 4(k-2)+3);
//   INT2 (channels at bits 2c): pair 2m+q holds (8q+m, 8q+4+m).
template <int BITS>
struct MagicPairs {
  static constexpr int kPairs = (BITS == 4) ? 4 : 8;
  uint32_t h[kPairs];
  // word channel of half e (0 = low) of pair k
  static constexpr int chan(int k, int e) {
    return (BITS == 4) ? ((k < 2) ? 4 * k + 2 * e : 4 * (k - 2) + 2 * e + 1) : 8 * ((k % 2)) + 4 * e + k / 2;
  }
  __device__ __forceinline__ MagicPairs(uint32_t w, uint32_t magic) {
    constexpr uint32_t kLo = 0x04010400u, kHi = 0x04030402u;  // bytes (0, 1) / (2, 3) under 0x64
    if constexpr (BITS == 4) {
      const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
      h[0] = __builtin_amdgcn_perm(magic, lo, kLo);
      h[1] = __builtin_amdgcn_perm(magic, lo, kHi);
      h[2] = __builtin_amdgcn_perm(magic, hi, kLo);
      h[3] = __builtin_amdgcn_perm(magic, hi, kHi);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t b = (w >> (2 * m)) & 0x03030303u;  // byte j = channel 4j + m
        h[2 * m] = __builtin_amdgcn_perm(magic, b, kLo);
        h[2 * m + 1] = __builtin_amdgcn_perm(magic, b, kHi);
      }
    }
  }
};

// channels per lane on the low-bit tier: 32 for single-head tiles (keys by
// integer dot products, so only the accumulators scale with it), 16 when the
// float q-hat of 2-4 heads is held too
constexpr int lowbit_cpl(int d, int rt) { return (rt == 1 ? 32 : 16) < d ? (rt == 1 ? 32 : 16) : d; }

// LDS of the per-tile key table: q-hat * scale [tiles][RT][D] and
// sum(q-hat * zero) [tiles][RT]; a low-bit split spans at most this many tiles.
constexpr int kKtLdsBytes = 24576;
constexpr int kt_max_tiles(int d, int rt) { return kKtLdsBytes / (4 * rt * (d + 1)); }

template <int D, int BITS, int RT, bool KT>
__device__ __forceinline__ void lowbit_split(const DecodeK& p, int unit, int n, int g, int tile, int split,
                                             const float* bvec, float* red, float (*sm)[RT], float* sM,
                                             float* po, float2* pml) {
  constexpr int CPL = lowbit_cpl(D, RT), LPT = D / CPL, SLOTS = kThreads / LPT, TPT = kTPTQ;
  constexpr int BATCH = SLOTS * TPT;
  constexpr int NB = CPL * BITS / 8, NW = NB / 4;  // code bytes / words per lane and token
  constexpr int CB = D * BITS / 8;                 // code bytes per token
  constexpr int CPW = 32 / BITS;                   // channels per code word
  constexpr bool kIntDot = (RT == 1) && !KT;
  static_assert(NB % 4 == 0 && NW >= 1 && NW <= 4, "lane code slice must be 1, 2 or 4 words");
  const int tid = threadIdx.x;
  const int lane = tid % LPT, tslot = tid / LPT, c0 = lane * CPL;
  const int gpt = D / p.group;
  const int gi = c0 / p.group;
  const int t0 = (split - p.S16) * p.Cq;
  const int t1 = min(p.nq, t0 + p.Cq);
  const int nt = max(t1 - t0, 0);  // tokens of this block (>= 1 for every planned split)
  const int64_t ub = static_cast<int64_t>(unit) * p.capq + t0;
  const uint32_t rbytes = static_cast<uint32_t>(nt) * CB;
  const uint32_t sbytes = static_cast<uint32_t>(nt) * gpt * 4;
  const Rsrc rk = make_rsrc(p.kq + ub * CB, rbytes);
  const Rsrc rv = make_rsrc(p.vq + ub * CB, rbytes);
  // per-channel key tiles have no per-token key (scale, zero)
  const Rsrc rks = make_rsrc(KT ? p.vsz + ub * gpt : p.ksz + ub * gpt, KT ? 0u : sbytes);
  const Rsrc rvs = make_rsrc(p.vsz + ub * gpt, sbytes);
  // byte offsets of this lane's slice of token 0 of its slot
  const uint32_t cof = static_cast<uint32_t>(tslot * CB + lane * NB);
  const uint32_t sof = static_cast<uint32_t>((tslot * gpt + gi) * 4);
  struct Regs { Words<NW> k[TPT], v[TPT]; uint32_t ks[TPT], vs[TPT]; };
  // base: first token of the batch, relative to t0
  auto load = [&](int base, Regs& R) {
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const uint32_t t = static_cast<uint32_t>(base + j * SLOTS);
      R.k[j] = bload<NW>(rk, cof + t * CB);
      if constexpr (!KT) R.ks[j] = bload1(rks, sof + t * gpt * 4);
      else R.ks[j] = 0u;
      R.v[j] = bload<NW>(rv, cof + t * CB);
      R.vs[j] = bload1(rvs, sof + t * gpt * 4);
    }
  };
  Regs A, B;
  load(0, A);
  float qh[RT][KT ? 1 : CPL];
  float qsum[RT];
  // per-channel key tiles: table of q-hat * scale and sum(q-hat * zero) of
  // the block's tiles (the range starts on a tile and holds whole tiles);
  // wave w builds tiles w, w + 4, ..., lane l channels l, l + 64
  __shared__ float kt_qs[KT ? kt_max_tiles(D, RT) * RT * D : 1];
  __shared__ float kt_qz[KT ? kt_max_tiles(D, RT) * RT : 1];
  const int ntl = nt / kKeyTile;
  if constexpr (KT) {
    constexpr int CPX = D / kWave;
    const int wave = tid / kWave, wl = tid % kWave;
    const float qscale = kLog2e / sqrtf(static_cast<float>(D));
    float qx[RT][CPX];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int h = g * p.rep + tile * RT + r;
      const uint16_t* qp = p.q + (static_cast<int64_t>(n) * p.hq + h) * D;
#pragma unroll
      for (int e = 0; e < CPX; ++e) {
        const int c = wl + e * kWave;
        qx[r][e] = h2f(qp[c]) * __builtin_amdgcn_rcpf(bvec[c]) * qscale;
      }
    }
    const uint32_t* zs = p.kcsz + (static_cast<int64_t>(unit) * (p.capq / kKeyTile) + t0 / kKeyTile) * D;
    for (int tl = wave; tl < ntl; tl += kThreads / kWave) {
      uint32_t w[CPX];
#pragma unroll
      for (int e = 0; e < CPX; ++e) w[e] = zs[static_cast<int64_t>(tl) * D + wl + e * kWave];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        float zsum = 0.0f;
#pragma unroll
        for (int e = 0; e < CPX; ++e) {
          kt_qs[(tl * RT + r) * D + wl + e * kWave] = qx[r][e] * lo_h(w[e]);
          zsum += qx[r][e] * hi_h(w[e]);
        }
        zsum = wave_sum(zsum);
        if (wl == 0) kt_qz[tl * RT + r] = zsum;
      }
    }
    __syncthreads();
  } else {
    load_qhat<D, RT, CPL>(p, n, g, tile, c0, bvec, qh);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      qsum[r] = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) qsum[r] += qh[r][i];
    }
  }
  // Integer form of q-hat (single head): q_int = rint(q-hat * 2^F) with F
  // chosen per lane so |q_int| < 2^22, biased by 2^23 into [0, 2^24) and
  // cut into six 4-bit digits laid out like the code nibbles. Then
  //   sum_c q_int[c]*code[c] = sum_d 16^d dot8(codes, digit_d)
  //                            - 2^23 * dot8(codes, 0x11111111),
  // exact in 32-bit integers (two's-complement wraparound cancels the bias).
  constexpr int NQW = CPL / 8;  // nibble words (8 channels each) per lane
  uint32_t qd[6][kIntDot ? NQW : 1];
  float qunit = 1.0f;
  if constexpr (kIntDot) {
    // |sum_c q_int*code| <= CPL * (2^BITS - 1) * 2^22 must fit a signed 32-bit
    // integer; the digit sums themselves may wrap, the result is taken mod 2^32
    static_assert(static_cast<long long>(CPL) * ((1 << BITS) - 1) * (1ll << 22) < (1ll << 31),
                  "the lane's dot product must fit 32 bits");
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) mx = fmaxf(mx, fabsf(qh[0][i]));
    int e = 0;
    if (mx > 0.0f) (void)frexpf(mx, &e);
    const int F = 22 - e;
    qunit = ldexpf(1.0f, -F);
#pragma unroll
    for (int d = 0; d < 6; ++d)
#pragma unroll
      for (int i = 0; i < NQW; ++i) qd[d][i] = 0;
#pragma unroll
    for (int i = 0; i < NQW; ++i) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // channel of nibble k in nibble word i
        int ch;
        if constexpr (BITS == 4) ch = 8 * i + k;
        else ch = 16 * (i / 2) + 2 * k + (i % 2);
        const int qi = static_cast<int>(rintf(ldexpf(qh[0][ch], F)));
        const uint32_t qb = static_cast<uint32_t>(qi + (1 << 23));
#pragma unroll
        for (int d = 0; d < 6; ++d) qd[d][i] |= ((qb >> (4 * d)) & 0xFu) << (4 * k);
      }
    }
  }
  Acc<RT, CPL> st;
  st.init();
  const uint32_t magic = opaque(0x64646464u);  // kept in a register for v_perm
  // one batch: TPT tokens per thread, token j of the slot at base + j*SLOTS
  auto step = [&](const Regs& R, int base) {
    float sc[TPT][RT];
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const bool valid = base + j * SLOTS + tslot < nt;
      const float s = lo_h(R.ks[j]), z = hi_h(R.ks[j]);
      if constexpr (KT) {
        // the token's tile (clamped for masked tokens past the range)
        const int tl = min((base + j * SLOTS + tslot) / kKeyTile, ntl - 1);
        float cf[CPL];
        unpack_codes<BITS, CPL>(R.k[j].w, cf);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const float* qs = kt_qs + (tl * RT + r) * D + c0;
          float dot = 0.0f;
#pragma unroll
          for (int i = 0; i < CPL; ++i) dot += qs[i] * cf[i];
          const float v = group_sum<LPT>(dot) + kt_qz[tl * RT + r];
          sc[j][r] = valid ? v : -INFINITY;
        }
      } else if constexpr (kIntDot) {
        uint32_t acc[6] = {0u, 0u, 0u, 0u, 0u, 0u}, csum = 0u;
#pragma unroll
        for (int i = 0; i < NQW; ++i) {
          uint32_t x;
          if constexpr (BITS == 4) x = R.k[j].w[i];
          else x = (i % 2 == 0) ? (R.k[j].w[i / 2] & 0x33333333u) : ((R.k[j].w[i / 2] >> 2) & 0x33333333u);
#pragma unroll
          for (int d = 0; d < 6; ++d) acc[d] = __builtin_amdgcn_udot8(x, qd[d][i], acc[d], false);
          csum = __builtin_amdgcn_udot8(x, 0x11111111u, csum, false);
        }
        const uint32_t u = acc[0] + (acc[1] << 4) + (acc[2] << 8) + (acc[3] << 12) +
                           (acc[4] << 16) + (acc[5] << 20);
        const int32_t rdot = static_cast<int32_t>(u - (csum << 23));
        const float dot = static_cast<float>(rdot) * qunit;
        const float v = group_sum<LPT>(s * dot + z * qsum[0]);
        sc[j][0] = valid ? v : -INFINITY;
      } else {
        float cf[CPL];
        unpack_codes<BITS, CPL>(R.k[j].w, cf);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          float dot = 0.0f;
#pragma unroll
          for (int i = 0; i < CPL; ++i) dot += qh[r][i] * cf[i];
          const float v = group_sum<LPT>(s * dot + z * qsum[r]);
          sc[j][r] = valid ? v : -INFINITY;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float bm = sc[0][r];
#pragma unroll
      for (int j = 1; j < TPT; ++j) bm = fmaxf(bm, sc[j][r]);
      st.rebase(r, bm);
    }
    float mref[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) mref[r] = fmaxf(st.m[r], -FLT_MAX);  // exp2(-inf - mref) = 0
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const float s = lo_h(R.vs[j]), z = hi_h(R.vs[j]);
      // value codes as fp16 1024 + code: a += w * (1024 + code), and the
      // 1024 * w it adds is taken back out of the zero-point sum z
      float w[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const float pr = fast_exp2(sc[j][r] - mref[r]);
        st.l[r] += pr;
        w[r] = pr * s;
        st.z[r] += pr * z;
        st.z[r] -= 1024.0f * w[r];
      }
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const MagicPairs<BITS> mp(R.v[j].w[i], magic);
#pragma unroll
        for (int k = 0; k < MagicPairs<BITS>::kPairs; ++k) {
          const float lo = lo_h(mp.h[k]), hi = hi_h(mp.h[k]);
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            st.a[r][CPW * i + MagicPairs<BITS>::chan(k, 0)] += w[r] * lo;
            st.a[r][CPW * i + MagicPairs<BITS>::chan(k, 1)] += w[r] * hi;
          }
        }
      }
    }
  };
  // two register sets in turn: the loads of one batch are in flight while
  // the other is computed
  for (int base = 0;;) {
    load(base + BATCH, B);
    step(A, base);
    base += BATCH;
    if (base >= nt) break;
    load(base + BATCH, A);
    step(B, base);
    base += BATCH;
    if (base >= nt) break;
  }
  write_partial<D, RT, LPT, CPL>(st, red, sm, sM, po, pml);
}

// ---------------------------------------------------------------------------
// FP16 tier: LPT lanes per token, CPL channels (2*CPL bytes) of the key and
// value rows per lane. Rows are read through a buffer resource spanning the
// block's slot range [s0, s1), as on the low-bit tier. The new token enters
// the state of the block that owns the free slot directly (the tile-0 block
// also writes its balanced key and value into that slot).
#ifndef MIKV_FP16_CPL1
#define MIKV_FP16_CPL1 8
#endif
#ifndef MIKV_FP16_TPT1
#define MIKV_FP16_TPT1 2
#endif
constexpr int fp16_cpl(int rt) { return rt == 1 ? MIKV_FP16_CPL1 : 8; }

// With per-channel key tiles (KT) the split after the low-bit splits streams
// the fp16 buffer of pairs that wait for a tile: the same arithmetic, with no
// FP16-tier scores to keep and no new token.
template <int D, int RT, bool KT>
__device__ __forceinline__ void fp16_split(const DecodeK& p, int unit, int n, int g, int tile, int split,
                                           const float* bvec, float* red, float (*sm)[RT], float* sM,
                                           float* po, float2* pml) {
  constexpr int CPL = fp16_cpl(RT), LPT = D / CPL, SLOTS = kThreads / LPT;
  constexpr int TPT = (RT == 1) ? MIKV_FP16_TPT1 : kTPT16;
  constexpr int BATCH = SLOTS * TPT;
  constexpr int NV = CPL / 8;  // 16-byte loads per row and lane
  const int tid = threadIdx.x;
  const int lane = tid % LPT, tslot = tid / LPT, c0 = lane * CPL;
  const bool buf = KT && split >= p.S16 + p.Sq;
  const int s0 = buf ? 0 : split * p.C16;
  const int s1 = buf ? p.nb : min(p.cap16, s0 + p.C16);
  const int ns = max(s1 - s0, 0);
  const int fr = buf ? -1 : p.free16[unit];
  const int64_t rb = static_cast<int64_t>(unit) * p.cap16;
  const uint32_t rbytes = static_cast<uint32_t>(ns) * D * 2;
  const int64_t bb = static_cast<int64_t>(unit) * kKeyTile * D;
  const Rsrc rk = make_rsrc(buf ? p.kbuf + bb : p.k16 + (rb + s0) * D, rbytes);
  const Rsrc rv = make_rsrc(buf ? p.vbuf + bb : p.v16 + (rb + s0) * D, rbytes);
  // scores of this tile's heads for the block's slots, [RT][cap16] rows
  const int64_t scb = (static_cast<int64_t>(unit) * p.rep + tile * RT) * p.cap16 + s0;
  const uint32_t cof = static_cast<uint32_t>((tslot * D + c0) * 2);
  struct Regs { Words<4> k[TPT][NV], v[TPT][NV]; };
  auto load = [&](int base, Regs& R) {
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const uint32_t off = cof + static_cast<uint32_t>(base + j * SLOTS) * (D * 2);
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        R.k[j][e] = bload<4>(rk, off + 16 * e);
        R.v[j][e] = bload<4>(rv, off + 16 * e);
      }
    }
  };
  Regs A, B;
  load(0, A);
  float qh[RT][CPL];
  load_qhat<D, RT, CPL>(p, n, g, tile, c0, bvec, qh);
  Acc<RT, CPL> st;
  st.init();
  // The new token: balanced key (fp32 product rounded once to fp16) and
  // value. In the block owning the free slot it seeds the state of slot
  // group 0 (max = its score, sum = 1, o = its value); the free slot's stale
  // row is masked in the stream (it holds finite values: zeros after the
  // prefill build, the demoted token's row after a decode step).
  const int frel = fr - s0;
  const bool owns_fr = frel >= 0 && frel < ns;
  if (owns_fr) {  // uniform
    const int64_t nb = static_cast<int64_t>(unit) * D + c0;
    uint4 kn[NV], vn[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      float kx[8];
      load8(p.k_new + nb + 8 * e, kx);
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = f2h(mul_rn(kx[2 * i], bvec[c0 + 8 * e + 2 * i]));
        const uint32_t hi = f2h(mul_rn(kx[2 * i + 1], bvec[c0 + 8 * e + 2 * i + 1]));
        w[i] = lo | (hi << 16);
      }
      kn[e] = make_uint4(w[0], w[1], w[2], w[3]);
      vn[e] = *reinterpret_cast<const uint4*>(p.v_new + nb + 8 * e);
      if (tile == 0 && tslot == 0) {
        *reinterpret_cast<uint4*>(p.k16 + (rb + fr) * D + c0 + 8 * e) = kn[e];
        *reinterpret_cast<uint4*>(p.v16 + (rb + fr) * D + c0 + 8 * e) = vn[e];
      }
    }
    if (tile == 0 && tid == 0) p.pos16[rb + fr] = p.len - 1;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kn[e]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dot += qh[r][8 * e + 2 * i] * lo_h(kw[i]);
          dot += qh[r][8 * e + 2 * i + 1] * hi_h(kw[i]);
        }
      }
      dot = group_sum<LPT>(dot);
      if (tslot == 0) {
        st.m[r] = dot;
        st.l[r] = 1.0f;
#pragma unroll
        for (int e = 0; e < NV; ++e) {
          const uint32_t* vw = reinterpret_cast<const uint32_t*>(&vn[e]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            st.a[r][8 * e + 2 * i] = lo_h(vw[i]);
            st.a[r][8 * e + 2 * i + 1] = hi_h(vw[i]);
          }
        }
        if (lane == 0) p.sc16[scb + static_cast<int64_t>(r) * p.cap16 + frel] = dot;
      }
    }
  }
  auto step = [&](const Regs& R, int base) {
    float sc[TPT][RT];
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int t = base + j * SLOTS + tslot;
      const bool valid = t < ns && t != frel;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < NV; ++e) {
          const uint32_t* kw = R.k[j][e].w;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dot += qh[r][8 * e + 2 * i] * lo_h(kw[i]);
            dot += qh[r][8 * e + 2 * i + 1] * hi_h(kw[i]);
          }
        }
        dot = group_sum<LPT>(dot);
        sc[j][r] = valid ? dot : -INFINITY;
        if (lane == 0 && valid && !buf) p.sc16[scb + static_cast<int64_t>(r) * p.cap16 + t] = dot;
      }
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float bm = sc[0][r];
#pragma unroll
      for (int j = 1; j < TPT; ++j) bm = fmaxf(bm, sc[j][r]);
      st.rebase(r, bm);
    }
    float mref[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) mref[r] = fmaxf(st.m[r], -FLT_MAX);
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      // masked rows (past the range: loaded as zeros; the stale free row:
      // finite) get probability 0 and add nothing
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const float pr = fast_exp2(sc[j][r] - mref[r]);
        st.l[r] += pr;
#pragma unroll
        for (int e = 0; e < NV; ++e) {
          const uint32_t* vw = R.v[j][e].w;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            st.a[r][8 * e + 2 * i] += pr * lo_h(vw[i]);
            st.a[r][8 * e + 2 * i + 1] += pr * hi_h(vw[i]);
          }
        }
      }
    }
  };
  if constexpr (RT == 1) {
    // three register sets in turn: two batches in flight while one is computed
    Regs C;
    load(BATCH, B);
    for (int base = 0;;) {
      load(base + 2 * BATCH, C);
      step(A, base);
      base += BATCH;
      if (base >= ns) break;
      load(base + 2 * BATCH, A);
      step(B, base);
      base += BATCH;
      if (base >= ns) break;
      load(base + 2 * BATCH, B);
      step(C, base);
      base += BATCH;
      if (base >= ns) break;
    }
  } else {
    // head tiles hold more state: two register sets
    for (int base = 0;;) {
      load(base + BATCH, B);
      step(A, base);
      base += BATCH;
      if (base >= ns) break;
      load(base + BATCH, A);
      step(B, base);
      base += BATCH;
      if (base >= ns) break;
    }
  }
  write_partial<D, RT, LPT, CPL>(st, red, sm, sM, po, pml);
}

template <int D, int BITS, int RT, bool KT>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(const DecodeK p) {
  // Split-major block order. Blocks are dispatched to the 8 XCDs in turn
  // (block i to XCD i mod 8), so with the split index outermost every XCD
  // sees consecutive (unit, tile) pairs of every split: the same mix of
  // FP16 and low-bit splits, instead of XCDs that hold only one tier's
  // splits and finish at different times. The tier whose blocks take
  // longer is dispatched first: a compute unit's older waves win issue.
  const int S = p.S16 + p.Sq + p.Sb;
  const int ut = p.units * p.tiles;
  const int sd = blockIdx.x / ut;
  // the buffer split (per-channel key tiles) comes last
  const int split = (sd >= p.S16 + p.Sq || p.f16_first) ? sd : ((sd < p.Sq) ? p.S16 + sd : sd - p.Sq);
  const int rest = blockIdx.x % ut;
  const int tile = rest % p.tiles;
  const int unit = rest / p.tiles;
  const int n = unit / p.hkv;
  const int g = unit % p.hkv;
  const float* bvec = p.b + static_cast<int64_t>(unit) * D;
  const int part = (unit * p.tiles + tile) * S + split;
  float* po = p.part_o + static_cast<int64_t>(part) * RT * D;
  float2* pml = p.part_ml + static_cast<int64_t>(part) * RT;

  __shared__ float red[4 * RT * D + 4 * RT];
  __shared__ float sm_max[4][RT];
  __shared__ float sm_M[RT];

  if (split < p.S16 || (KT && split >= p.S16 + p.Sq)) {
    fp16_split<D, RT, KT>(p, unit, n, g, tile, split, bvec, red, sm_max, sm_M, po, pml);
  } else {
    lowbit_split<D, BITS, RT, KT>(p, unit, n, g, tile, split, bvec, red, sm_max, sm_M, po, pml);
  }
}

#include "decode_tile.hpp"

// Grid: (unit, output chunk [+ 1]). An output block of unit x combines the
// split partials of kMergeOut * G outputs (head, channel) of the unit,
// kMergeTPO threads per output, each summing a strided subset of the splits,
// so a unit with many splits spreads its partials over many blocks and
// loads. One block per unit turns the FP16-tier scores into p16 and, when
// FUSE, applies the decode-step H2O update (acc += p16, drop the worst
// candidate, demote it), which the stand-alone H2O kernel would otherwise do
// in a third launch. That is an extra block beside the output blocks when
// the grid stays within one wave of blocks (32K GQA: step 43.4 -> 40.9 us),
// else output block 0 after its outputs (a 1536-block grid cost the GQA
// batch about 1 us).
// Dynamic LDS: [rep][S] (max, sum) pairs, then [rep] maxima and [rep]
// reciprocal sums.
constexpr int kMergeOut = 64;
constexpr int kMergeTPO = kThreads / kMergeOut;
constexpr int kMergeSlots = 16;  // FP16-tier slots per thread held in registers
constexpr int kMergeHeads = 4;   // heads whose FP16-tier scores are loaded up front

#ifndef MIKV_MERGE_MAX_BLOCKS
#define MIKV_MERGE_MAX_BLOCKS 1024
#endif
constexpr long kMergeMaxBlocks = MIKV_MERGE_MAX_BLOCKS;  // above this, one block takes several output groups
template <int D, int BITS, int NL, bool FUSE, int G>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(const DecodeK p, int RT, H2OView hv, bool sep) {
  extern __shared__ float2 sml[];
  __shared__ float red[kThreads];
  const int unit = blockIdx.x;
  const int chunk = blockIdx.y;
  const int n = unit / p.hkv, g = unit % p.hkv;
  const int tid = threadIdx.x;
  const int S = p.S16 + p.Sq + p.Sb;
  const int rep = p.rep;
  const int cap16 = p.cap16;
  float* sM = reinterpret_cast<float*>(sml + rep * S);
  float* sIL = sM + rep;
  const float2* __restrict__ pml = p.part_ml;
  const float* __restrict__ pov = p.part_o;
  const float* __restrict__ sc = p.sc16 + static_cast<int64_t>(unit) * rep * cap16;
  const int64_t base16 = static_cast<int64_t>(unit) * cap16;
  // With sep, the unit's last block (chunk gridDim.y - 1) turns the FP16-tier
  // scores into p16 and applies the H2O update while the others combine the
  // outputs, side by side; without it, block 0 does both, one after the other.
  const bool last = chunk == static_cast<int>(gridDim.y) - 1;
  const bool do_out = !(sep && last);
  const bool pblk = sep ? last : chunk == 0;
  // heads this block needs (statistics): its outputs' heads, or all for p16
  const int out0 = chunk * kMergeOut * G;
  const int h_lo = pblk ? 0 : out0 / D;
  const int h_hi = pblk ? rep : min(rep, (out0 + kMergeOut * G - 1) / D + 1);
  // (1) issue every load before the first wait: the thread's partial
  // outputs, the FP16-tier scores of up to kMergeHeads heads and the H2O
  // state (chunk 0), then the split statistics, whose LDS stores wait for
  // all of them at once
  // group gi of the block: outputs out0 + 64*gi + (tid % 64)
  const int sub = tid / kMergeOut;  // the thread's subset of splits: s = sub, sub + TPO, ...
  auto out_of = [&](int gi) { return out0 + gi * kMergeOut + tid % kMergeOut; };
  auto part_of = [&](int oi) {
    const int hl = oi / D;
    return pov + (static_cast<int64_t>((unit * p.tiles + hl / RT) * S) * RT + hl % RT) * D + oi % D;
  };
  constexpr int PF = (G == 1) ? 8 : 2;  // splits per thread loaded up front, per group
  float pf[G][PF];
  if (do_out) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int oi = out_of(gi);
      const float* po = part_of(oi < rep * D ? oi : 0);
#pragma unroll
      for (int k = 0; k < PF; ++k) {
        const int s = sub + k * kMergeTPO;
        pf[gi][k] = (oi < rep * D && s < S) ? po[static_cast<int64_t>(s) * RT * D] : 0.0f;
      }
    }
  }
  const bool slots_in_regs = cap16 <= kMergeSlots * kThreads;
  float sv[kMergeHeads][kMergeSlots], accv[kMergeSlots];
  int posv[kMergeSlots];
  int fr = 0;
  // slot rounds actually used; heads and rounds are uniform branches, and
  // slot indices past the tier are clamped (their values are never used),
  // so the loads issue back to back without per-lane branches
  const int nslot = (cap16 + kThreads - 1) / kThreads;
  if (pblk) {
    if (slots_in_regs) {
#pragma unroll
      for (int h = 0; h < kMergeHeads; ++h) {
        if (h < rep) {
#pragma unroll
          for (int k = 0; k < kMergeSlots; ++k)
            if (k < nslot) sv[h][k] = sc[h * cap16 + min(tid + k * kThreads, cap16 - 1)];
        }
      }
    }
    if constexpr (FUSE) {
      fr = hv.free16[unit];
#pragma unroll
      for (int k = 0; k < kMergeSlots; ++k) {
        if (k < nslot) {
          const int sl = min(tid + k * kThreads, cap16 - 1);
          accv[k] = hv.acc16[base16 + sl];
          posv[k] = hv.pos16[base16 + sl];
        }
      }
    }
  }
  for (int i = h_lo * S + tid; i < h_hi * S; i += kThreads) {
    const int hl = i / S, s = i % S;
    sml[i] = pml[(static_cast<int64_t>((unit * p.tiles + hl / RT) * S) + s) * RT + hl % RT];
  }
  __syncthreads();
  // (2) per head: maximum and reciprocal normaliser, one wave per head, its
  // lanes taking the splits in turn (a unit of a long sequence has ~64)
  {
    const int wave = tid / kWave, lane = tid % kWave;
    for (int hl = h_lo + wave; hl < h_hi; hl += kThreads / kWave) {
      float M = -INFINITY;
      for (int s = lane; s < S; s += kWave) M = fmaxf(M, sml[hl * S + s].x);
      M = wave_max(M);
      float L = 0.0f;
      for (int s = lane; s < S; s += kWave) L += sml[hl * S + s].y * fast_exp2(sml[hl * S + s].x - M);
      L = wave_sum(L);
      if (lane == 0) {
        sM[hl] = M;
        sIL[hl] = 1.0f / L;
      }
    }
  }
  __syncthreads();
  // (3) outputs: each thread sums its subset of splits, then the kMergeTPO
  // threads of an output combine through LDS
  if (do_out) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int oi = out_of(gi);
      const bool has_out = oi < rep * D;
      const int ohl = oi / D, oc = oi % D;
      float v = 0.0f;
      if (has_out) {
        const float M = sM[ohl];
        const float2* ml = sml + ohl * S;
#pragma unroll
        for (int k = 0; k < PF; ++k) {
          const int s = sub + k * kMergeTPO;
          if (s < S) v += pf[gi][k] * fast_exp2(ml[s].x - M);
        }
        const float* po = part_of(oi);
#pragma unroll 4
        for (int s = sub + PF * kMergeTPO; s < S; s += kMergeTPO)
          v += po[static_cast<int64_t>(s) * RT * D] * fast_exp2(ml[s].x - M);
      }
      if (gi > 0) __syncthreads();  // the previous group's reads of red are done
      red[tid] = v;
      __syncthreads();
      if (tid < kMergeOut && has_out) {
        float t = 0.0f;
#pragma unroll
        for (int k = 0; k < kMergeTPO; ++k) t += red[tid + k * kMergeOut];
        p.o[(static_cast<int64_t>(n) * p.hq + g * rep + ohl) * D + oc] = t * sIL[ohl];
      }
    }
  }
  if (!pblk) return;
  // (4) p16 = sum over the group's heads of the FP16-tier probabilities
  float* __restrict__ p16 = p.p16 + base16;
  auto prob = [&](int sl) {
    float a = 0.0f;
    for (int hl = 0; hl < rep; ++hl) a += fast_exp2(sc[hl * cap16 + sl] - sM[hl]) * sIL[hl];
    return a;
  };
  if (slots_in_regs) {
    // all loads of a head are issued together, before any store
    float pa[kMergeSlots];
#pragma unroll
    for (int k = 0; k < kMergeSlots; ++k)
      if (k < nslot) pa[k] = fast_exp2(sv[0][k] - sM[0]) * sIL[0];
#pragma unroll
    for (int hl = 1; hl < kMergeHeads; ++hl) {
      if (hl < rep) {
        const float M = sM[hl], IL = sIL[hl];
#pragma unroll
        for (int k = 0; k < kMergeSlots; ++k)
          if (k < nslot) pa[k] += fast_exp2(sv[hl][k] - M) * IL;
      }
    }
    for (int hl = kMergeHeads; hl < rep; ++hl) {
      float x[kMergeSlots];
#pragma unroll
      for (int k = 0; k < kMergeSlots; ++k)
        if (k < nslot) x[k] = sc[hl * cap16 + min(tid + k * kThreads, cap16 - 1)];
      const float M = sM[hl], IL = sIL[hl];
#pragma unroll
      for (int k = 0; k < kMergeSlots; ++k)
        if (k < nslot) pa[k] += fast_exp2(x[k] - M) * IL;
    }
    Worst w;
    const int limit = hv.len - hv.recent;
#pragma unroll
    for (int k = 0; k < kMergeSlots; ++k) {
      const int sl = tid + k * kThreads;
      if (k < nslot && sl < cap16) {
        const float a = pa[k];
        p16[sl] = a;
        if constexpr (FUSE) {
          const float prev = (sl == fr) ? 0.0f : accv[k];
          const int pos = (sl == fr) ? hv.len - 1 : posv[k];
          const float v = prev + a;
          hv.acc16[base16 + sl] = v;
          if (pos < limit) w.consider(v, pos, sl);
        }
      }
    }
    if constexpr (FUSE) h2o_select_demote<D, BITS, NL>(w, hv, unit);
  } else {
    for (int sl = tid; sl < cap16; sl += kThreads) p16[sl] = prob(sl);
  }
}

static inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Compute units of the current device (the grid is sized to one resident
// round of blocks over all of them), read once per device and cached; 256
// (MI355X) when no device answers.
static int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      return 256;
    }
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Resident split-kernel blocks per compute unit for this instantiation, from
// the runtime's occupancy calculator (cached per instantiation); the
// default when it cannot answer (no device).
template <int D, int BITS, int IB, int RT, bool TILE, bool KT = false>
static const void* split_kernel_ptr() {
  if constexpr (TILE) return reinterpret_cast<const void*>(decode_tile_kernel<D, BITS, IB, RT>);
  else return reinterpret_cast<const void*>(decode_split_kernel<D, BITS, RT, KT>);
}
template <int D, int BITS, int IB, int RT, bool TILE, bool KT = false>
static int blocks_per_cu() {
  constexpr int kCap = (TILE && tile_mv<D, BITS, RT>()) ? kMvBlocksPerCU : MIKV_BLOCKS_PER_CU;
  static std::atomic<int> cache{0};
  int n = cache.load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, split_kernel_ptr<D, BITS, IB, RT, TILE, KT>(), kThreads,
                                                     0) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      return kCap;
    }
    cache.store(n, std::memory_order_relaxed);
  }
  return n < kCap ? n : kCap;
}
// decode_tile_kernel (scores on the matrix cores) for head tiles of 2-4
// heads, and for every tile when the importance tier holds codes; groups of
// d/2 channels. Otherwise decode_split_kernel.
static inline bool use_tile_kernel(int d, int group, int rt, int ib, int key_tile) {
  return key_tile == 0 && group == d / 2 && (ib < 16 || rt > 1);
}
static int split_blocks_per_cu(int d, int bits, int ib, int rt, bool tile, int key_tile) {
#define MIKV_OCCK(D_, B_)                                      \
  if (key_tile && d == D_ && bits == B_) {                     \
    if (rt == 1) return blocks_per_cu<D_, B_, 16, 1, false, true>(); \
    if (rt == 2) return blocks_per_cu<D_, B_, 16, 2, false, true>(); \
    return blocks_per_cu<D_, B_, 16, 4, false, true>();        \
  }
  MIKV_OCCK(128, 4) MIKV_OCCK(128, 2) MIKV_OCCK(64, 4) MIKV_OCCK(64, 2)
#undef MIKV_OCCK
#define MIKV_OCC16(D_, B_, RT_)                           \
  if (d == D_ && bits == B_ && ib == 16 && rt == RT_)     \
    return tile ? blocks_per_cu<D_, B_, 16, RT_, (RT_ > 1)>() : blocks_per_cu<D_, B_, 16, RT_, false>();
#define MIKV_OCCQ(D_, B_, IB_)                                                           \
  if (d == D_ && bits == B_ && ib == IB_) {                                              \
    if (rt == 1) return blocks_per_cu<D_, B_, IB_, 1, true>();                           \
    if (rt == 2) return blocks_per_cu<D_, B_, IB_, 2, true>();                           \
    return blocks_per_cu<D_, B_, IB_, 4, true>();                                        \
  }
  MIKV_OCC16(128, 4, 1) MIKV_OCC16(128, 4, 2) MIKV_OCC16(128, 4, 4)
  MIKV_OCC16(128, 2, 1) MIKV_OCC16(128, 2, 2) MIKV_OCC16(128, 2, 4)
  MIKV_OCC16(64, 4, 1) MIKV_OCC16(64, 4, 2) MIKV_OCC16(64, 4, 4)
  MIKV_OCC16(64, 2, 1) MIKV_OCC16(64, 2, 2) MIKV_OCC16(64, 2, 4)
  MIKV_OCCQ(128, 4, 8) MIKV_OCCQ(128, 4, 4) MIKV_OCCQ(128, 2, 8) MIKV_OCCQ(128, 2, 4)
  MIKV_OCCQ(64, 4, 8) MIKV_OCCQ(64, 4, 4) MIKV_OCCQ(64, 2, 8) MIKV_OCCQ(64, 2, 4)
#undef MIKV_OCC16
#undef MIKV_OCCQ
  return MIKV_BLOCKS_PER_CU;
}

// Split sizes. The grid is sized to one resident wave of blocks
// (the instantiation's occupancy, at most MIKV_BLOCKS_PER_CU per compute
// unit), so no block starts after the others have drained. The
// splits of a (sequence, kv head) are shared between the tiers in
// proportion to the time their tokens take, so blocks end together; each
// tier gets at least one split when it has tokens. Single-head tiles are
// bound by HBM: the time of a tier is its bytes. Tiles of 2-4 heads are
// bound by VALU issue, and a token costs about the same instructions in
// both tiers (4 heads x d multiply-adds for the score and as many for the
// value sum; the low-bit unpacking roughly matches the FP16 tier's wider
// lane groups): the time of a tier is its token count, an FP16 token
// weighted 1.3 (on the 32K GQA shape, token shares of 1:1 and 1.3:1 gave a
// split kernel of 29.6 and 28.7 us, byte shares 34.2 us; the GQA batch, one
// split per tier and unit, takes the same plan at any weight), and 2.4 where
// the low-bit tier's value sums run on the matrix cores, which makes its
// tokens cheaper (32K GQA shape: 17.8 us at 1.2, 17.4-17.5 at 1.6, 16.8-17.1
// at 2.0-3.0; splits rounded to whole 256-token steps, which makes the FP16
// splits longer: 19.0 us).
//
// Per-channel key tiles: the low-bit splits hold whole tiles of 64 tokens
// (at most kt_max_tiles, the LDS table of a block), and the buffered pairs,
// if any, are one more split (Sb = 1) whose bytes count with the FP16 tier.
DecodePlan decode_plan(int batch, int hkv, int d, int bits, int group, int rep, int cap16, int nr,
                       int imp_bits, int key_tile) {
  DecodePlan pl;
  pl.RT = (rep % 4 == 0) ? 4 : (rep % 2 == 0 ? 2 : 1);
  pl.tiles = rep / pl.RT;
  pl.key_tile = key_tile;
  const int nq = key_tile ? nr / kKeyTile * kKeyTile : nr;
  pl.nq = nq;
  pl.nb = nr - nq;
  pl.Sb = pl.nb > 0 ? 1 : 0;
  const bool tile = use_tile_kernel(d, group, pl.RT, imp_bits, key_tile);
  const double b16 = static_cast<double>(cap16) *
                     (imp_bits == 16 ? 4.0 * d : 2.0 * (d * imp_bits / 8 + 4 * (d / group)));
  const double bq = static_cast<double>(nq) * 2.0 * (d * bits / 8 + 4 * (d / group));
  // a code importance tier costs like the retained tier: shares by bytes
  const double w16 = (tile && tile_mv_of(d, bits, pl.RT)) ? 2.4 : 1.3;
  const double t16 = (pl.RT == 1 || imp_bits < 16) ? b16 : w16 * cap16;
  const double tq = (pl.RT == 1 || imp_bits < 16) ? bq : static_cast<double>(nq);
  const long units = static_cast<long>(batch) * hkv * pl.tiles;
  long per_unit =
      (static_cast<long>(device_cus()) * split_blocks_per_cu(d, bits, imp_bits, pl.RT, tile, key_tile)) / units;
  // no split below ~16 KB of rows
  const long cap_splits = static_cast<long>((b16 + bq) / 16384.0) + 1;
  if (per_unit > cap_splits) per_unit = cap_splits;
  // Dispatch order. Two blocks share a compute unit and the older one wins
  // issue, so the tier with the longer blocks goes first. That is the
  // low-bit tier for single-head tiles, and also for head tiles whose grid
  // needs two rounds (the FP16 blocks then fill the second round). With one
  // round of head-tile blocks the FP16 blocks are the long ones: an FP16
  // token costs about 1.6 low-bit tokens there (per-block timestamps, 32K
  // GQA shape: FP16-first 27.2 us against 28.1 us; GQA batch FP16-first
  // 85.5 us against 81.1 us; 4K MHA layer 43.1 against 40.8 us).
  pl.f16_first = (pl.RT > 1 && imp_bits == 16 && per_unit >= 2) ? 1 : 0;
  if (nq > 0) {
    if (per_unit < 2) per_unit = 2;
    long s16 = static_cast<long>(per_unit * t16 / (t16 + tq) + 0.5);
    if (s16 < 1) s16 = 1;
    if (s16 > per_unit - 1) s16 = per_unit - 1;
    if (s16 > cap16) s16 = cap16;
    long sq = per_unit - s16;
    if (sq > nq) sq = nq;
    pl.S16 = static_cast<int>(s16);
    pl.Sq = static_cast<int>(sq);
  } else {
    pl.S16 = static_cast<int>(per_unit < 1 ? 1 : (per_unit > cap16 ? cap16 : per_unit));
    pl.Sq = 0;
  }
  pl.C16 = cdiv(cap16, pl.S16);
  pl.S16 = cdiv(cap16, pl.C16);
  pl.Cq = nq > 0 ? cdiv(nq, pl.Sq) : 0;
  if (nq > 0 && key_tile) {
    // whole tiles per split, within the block's LDS table
    const int mt = (d == 128) ? (pl.RT == 1 ? kt_max_tiles(128, 1) : pl.RT == 2 ? kt_max_tiles(128, 2)
                                                                                : kt_max_tiles(128, 4))
                              : (pl.RT == 1 ? kt_max_tiles(64, 1) : pl.RT == 2 ? kt_max_tiles(64, 2)
                                                                               : kt_max_tiles(64, 4));
    pl.Cq = cdiv(pl.Cq, kKeyTile) * kKeyTile;
    if (pl.Cq > mt * kKeyTile) pl.Cq = mt * kKeyTile;
  }
  if (nq > 0) pl.Sq = cdiv(nq, pl.Cq);
  return pl;
}

static inline size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t decode_ws_bytes(int batch, int hq, int hkv, int d, int cap16, const DecodePlan& pl) {
  const size_t units = static_cast<size_t>(batch) * hkv;
  const size_t rep = hq / hkv;
  const size_t nparts = units * pl.tiles * (pl.S16 + pl.Sq + pl.Sb);
  return al256(nparts * pl.RT * sizeof(float2)) + al256(nparts * pl.RT * d * sizeof(float)) +
         al256(units * rep * cap16 * sizeof(float));
}

// Workspace for every length up to nr_max: the partial count of any plan is
// at most max(4, blocks-per-unit) + 1 splits per (sequence, kv head, tile)
// (head tiles take up to 4 splits when fewer than two blocks per unit fit),
// plus the buffer split of per-channel key tiles, plus the low-bit splits that
// the LDS table of per-channel key tiles may add (one per kt_max_tiles tiles).
size_t decode_ws_bound(int batch, int hq, int hkv, int d, int bits, int group, int cap16, int nr_max,
                       int imp_bits, int key_tile) {
  const int rep = hq / hkv;
  DecodePlan pl = decode_plan(batch, hkv, d, bits, group, rep, cap16, nr_max, imp_bits, key_tile);
  const long units = static_cast<long>(batch) * hkv * pl.tiles;
  long per_unit = (static_cast<long>(device_cus()) * MIKV_BLOCKS_PER_CU) / units;
  if (per_unit < 4) per_unit = 4;
  long extra = 0;
  if (key_tile) extra = 1 + cdiv(nr_max, kt_max_tiles(d, 4) * kKeyTile);
  pl.S16 = static_cast<int>(per_unit + 1 + extra);
  pl.Sq = 0;
  pl.Sb = 0;
  return decode_ws_bytes(batch, hq, hkv, d, cap16, pl);
}

template <int D, int BITS, int IB, int RT, bool KT>
static hipError_t launch_da(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
  DecodeK k;
  k.hq = a.hq; k.hkv = a.hkv; k.rep = a.hq / a.hkv; k.cap16 = a.cap16; k.capq = a.capq;
  k.nq = pl.nq; k.len = a.len; k.group = a.group; k.units = a.batch * a.hkv;
  k.Sb = pl.Sb; k.nb = pl.nb;
  k.kcsz = reinterpret_cast<const uint32_t*>(a.kcsz);
  k.kbuf = a.kbuf; k.vbuf = a.vbuf;
  k.S16 = pl.S16; k.Sq = pl.Sq; k.C16 = pl.C16; k.Cq = pl.Cq; k.tiles = pl.tiles; k.f16_first = pl.f16_first;
  k.q = a.q; k.k_new = a.k_new; k.v_new = a.v_new; k.b = a.b;
  k.k16 = a.k16; k.v16 = a.v16; k.pos16 = a.pos16; k.free16 = a.free16;
  k.kq = a.kq; k.vq = a.vq;
  k.ksz = reinterpret_cast<const uint32_t*>(a.ksz);
  k.vsz = reinterpret_cast<const uint32_t*>(a.vsz);
  k.kimp = a.kimp; k.vimp = a.vimp;
  k.kimpsz = reinterpret_cast<uint32_t*>(a.kimpsz);
  k.vimpsz = reinterpret_cast<uint32_t*>(a.vimpsz);
  k.o = a.o; k.p16 = a.p16;
  const size_t units = static_cast<size_t>(a.batch) * a.hkv;
  const int S = pl.S16 + pl.Sq + pl.Sb;
  const size_t nparts = units * pl.tiles * S;
  char* w = static_cast<char*>(a.ws);
  k.part_ml = reinterpret_cast<float2*>(w);
  w += al256(nparts * pl.RT * sizeof(float2));
  k.part_o = reinterpret_cast<float*>(w);
  w += al256(nparts * pl.RT * D * sizeof(float));
  k.sc16 = reinterpret_cast<float*>(w);
  hipError_t e;
  // IB < 16 (a code importance tier): decode_tile_kernel for every tile;
  // IB = 16: the tile kernel for head tiles of groups d/2, else the split kernel
  constexpr bool kTileAlways = IB < 16;
  const bool tile = !KT && (kTileAlways || use_tile_kernel(D, a.group, RT, IB, 0));
  const void* kfn = tile ? split_kernel_ptr<D, BITS, IB, RT, (kTileAlways || RT > 1)>()
                         : split_kernel_ptr<D, BITS, IB, RT, false, KT>();
  if (a.ev_split_start || a.ev_split_stop) {
    // the events take the kernel's own start and end timestamps
    void* args[] = {&k};
    e = hipExtLaunchKernel(kfn, dim3(static_cast<unsigned>(nparts)), dim3(kThreads), args, 0, stream,
                           a.ev_split_start, a.ev_split_stop, 0);
  } else if (tile) {
    if constexpr (!KT && (kTileAlways || RT > 1))
      decode_tile_kernel<D, BITS, IB, RT><<<static_cast<unsigned>(nparts), kThreads, 0, stream>>>(k);
    e = hipGetLastError();
  } else {
    if constexpr (!kTileAlways)
      decode_split_kernel<D, BITS, RT, KT><<<static_cast<unsigned>(nparts), kThreads, 0, stream>>>(k);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  const size_t lds = static_cast<size_t>(k.rep) * S * sizeof(float2) + 2 * k.rep * sizeof(float);
  const bool fuse = !KT && a.fuse_h2o && a.cap16 <= kFusedMaxCap16;
  H2OView hv = a.h2o;
  if (!a.fuse_h2o) hv.len = a.len, hv.recent = 0;
  // Output groups of 64 per merge block: with few splits one block takes all
  // of a unit's outputs (fewer, fuller blocks); with many splits the outputs
  // spread over a 2-D grid so each block reads a bounded number of partials.
  const int groups = (k.rep * D + kMergeOut - 1) / kMergeOut;
  int G = 1;
  if (S <= 2 * kMergeTPO)
    while (G < 8 && G < groups && units * ((groups + G - 1) / G) > kMergeMaxBlocks) G *= 2;
  // Output chunks, plus one block per unit for p16 and the H2O update while
  // that still fits one wave of blocks; otherwise chunk 0 does that work too.
  const int chunks = (groups + G - 1) / G;
  const bool sep = units * (chunks + 1) <= kMergeMaxBlocks;
  const dim3 mgrid(static_cast<unsigned>(units), static_cast<unsigned>(chunks + (sep ? 1 : 0)));
#define MIKV_MERGE_G(NL_, F_, G_) \
  decode_merge_kernel<D, BITS, NL_, F_, G_><<<mgrid, kThreads, lds, stream>>>(k, RT, hv, sep)
#define MIKV_MERGE(NL_, F_)                   \
  do {                                        \
    if (G == 1) MIKV_MERGE_G(NL_, F_, 1);     \
    else if (G == 2) MIKV_MERGE_G(NL_, F_, 2); \
    else if (G == 4) MIKV_MERGE_G(NL_, F_, 4); \
    else MIKV_MERGE_G(NL_, F_, 8);            \
  } while (0)
  if (!fuse) MIKV_MERGE(D / 16, false);
  else if constexpr (!KT) {
    if (a.group == D / 2) MIKV_MERGE(D / 16, true);
    else MIKV_MERGE(D / 8, true);
  }
#undef MIKV_MERGE
#undef MIKV_MERGE_G
  return hipGetLastError();
}

hipError_t launch_decode_attn(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
  if (pl.key_tile) {
    if (a.imp_bits != 16) return hipErrorInvalidValue;
#define MIKV_DAK(D_, B_, RT_) \
    if (a.d == D_ && a.bits == B_ && pl.RT == RT_) return launch_da<D_, B_, 16, RT_, true>(a, pl, stream);
#define MIKV_DAK3(D_, B_) MIKV_DAK(D_, B_, 1) MIKV_DAK(D_, B_, 2) MIKV_DAK(D_, B_, 4)
    MIKV_DAK3(128, 4) MIKV_DAK3(128, 2) MIKV_DAK3(64, 4) MIKV_DAK3(64, 2)
#undef MIKV_DAK3
#undef MIKV_DAK
    return hipErrorInvalidValue;
  }
#define MIKV_DA(D_, B_, IB_, RT_) \
  if (a.d == D_ && a.bits == B_ && a.imp_bits == IB_ && pl.RT == RT_) return launch_da<D_, B_, IB_, RT_, false>(a, pl, stream);
#define MIKV_DA3(D_, B_, IB_) MIKV_DA(D_, B_, IB_, 1) MIKV_DA(D_, B_, IB_, 2) MIKV_DA(D_, B_, IB_, 4)
  MIKV_DA3(128, 4, 16) MIKV_DA3(128, 2, 16) MIKV_DA3(64, 4, 16) MIKV_DA3(64, 2, 16)
  if (a.group == a.d / 2) {
    MIKV_DA3(128, 4, 8) MIKV_DA3(128, 4, 4) MIKV_DA3(128, 2, 8) MIKV_DA3(128, 2, 4)
    MIKV_DA3(64, 4, 8) MIKV_DA3(64, 4, 4) MIKV_DA3(64, 2, 8) MIKV_DA3(64, 2, 4)
  }
#undef MIKV_DA3
#undef MIKV_DA
  return hipErrorInvalidValue;
}

}  // namespace mikv
