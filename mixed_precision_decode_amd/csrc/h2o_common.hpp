// Decode-step H2O bookkeeping shared by the stand-alone H2O kernel and the
// fused decode-step merge kernel (velog notes "No Token Left Behind ...",
// Key contributions 1): importance-based eviction decides the FP16 set and the
// evicted token is kept as low-bit codes; paperlayer summary of arXiv
// 2402.18096, section 5: heavy hitters plus local tokens).
#pragma once

#include "common.hpp"

namespace mikv {

struct H2OView {
  int cap16, capq, len, recent;
  int imp_bits;       // 16: fp16 importance tier (k16, v16); 8 or 4: codes
  uint16_t* k16;
  uint16_t* v16;
  uint8_t* kimp;      // importance tier as codes (IB < 16)
  uint8_t* vimp;
  uint32_t* kimpsz;   // (scale | zero << 16) per group
  uint32_t* vimpsz;
  int32_t* pos16;
  float* acc16;
  int32_t* free16;
  uint8_t* kq;
  uint8_t* vq;
  uint32_t* ksz;
  uint32_t* vsz;
  int32_t* posq;
  int32_t* demoted_pos;
  // per-channel key tiles (key_tile = 64): kq rows hold tiles of 64 tokens
  // whose (scale | zero << 16) words are kcsz [tile][d]; demoted pairs wait
  // in kbuf / vbuf [64][d] fp16 (positions posbuf) until a tile fills
  int key_tile;
  uint32_t* kcsz;
  uint16_t* kbuf;
  uint16_t* vbuf;
  int32_t* posbuf;
};

constexpr int kKeyTile = 64;

// Per-channel quantization of one tile of keys (velog notes "No Token Left
// Behind ...", the per-channel alternative and its appendix C summary;
// paperlayer summary of arXiv 2402.18096, appendix C: per-channel key
// quantization with groups of 64 along the tokens). xs: LDS [64][D] fp16
// rows of the tile, token-major; cl: LDS [64][D] bytes of scratch. Channel c
// is one quantization group of 64 values, held as 8 tokens by each of 8
// consecutive lanes, so quantize8_codes applies the per-token rule (same
// fixed fp32 sequence) along the tokens. The codes are packed token-major
// like per-token rows into kq_tile [64][D*BITS/8]; (scale | zero << 16) of
// channel c goes to kcsz_tile[c]. All 256 threads of the block call it.
template <int D, int BITS>
__device__ __forceinline__ void quantize_key_tile(const uint16_t* xs, uint8_t* cl, uint8_t* kq_tile,
                                                  uint32_t* kcsz_tile) {
  const int tid = threadIdx.x;
  const int l8 = tid % 8;  // tokens 8*l8 .. 8*l8 + 7 of the lane's channel
  static_assert(D % 32 == 0, "32 channels per pass");
  for (int c = tid / 8; c < D; c += 32) {  // the same trip count on every lane
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = h2f(xs[(8 * l8 + e) * D + c]);
    uint32_t szw, code[8];
    quantize8_codes<BITS, 8>(x, &szw, code);
#pragma unroll
    for (int e = 0; e < 8; ++e) cl[(8 * l8 + e) * D + c] = static_cast<uint8_t>(code[e]);
    if (l8 == 0) kcsz_tile[c] = szw;
  }
  __syncthreads();
  constexpr int CPW = 32 / BITS, WPR = D / CPW, CB = D * BITS / 8;
  for (int i = tid; i < kKeyTile * WPR; i += 256) {
    const int t = i / WPR, w = i % WPR;
    uint32_t word = 0;
#pragma unroll
    for (int m = 0; m < CPW; ++m) word |= static_cast<uint32_t>(cl[t * D + w * CPW + m]) << (BITS * m);
    reinterpret_cast<uint32_t*>(kq_tile + static_cast<int64_t>(t) * CB)[w] = word;
  }
}

// Per-token quantization of 64 value rows into the low-bit slots of a tile:
// rows t < 63 from vsrc [63][D] (global), row 63 from vlast; LPR = D/8 lanes
// per row, groups of NL lanes.
template <int D, int BITS, int NL>
__device__ __forceinline__ void quantize_value_tile(const uint16_t* vsrc, const uint16_t* vlast, uint8_t* vq_tile,
                                                    uint32_t* vsz_tile) {
  constexpr int LPR = D / 8, RPP = 256 / LPR, CB = D * BITS / 8, GPT = D / (8 * NL);
  const int tid = threadIdx.x, lane = tid % LPR;
  for (int t = tid / LPR; t < kKeyTile; t += RPP) {  // rows stay whole within a pass
    float x[8];
    load8((t < kKeyTile - 1 ? vsrc + static_cast<int64_t>(t) * D : vlast) + lane * 8, x);
    uint32_t szw;
    const uint32_t packed = quantize8<BITS, NL>(x, &szw);
    store_codes8<BITS>(vq_tile + static_cast<int64_t>(t) * CB, lane, packed);
    if (lane % NL == 0) vsz_tile[t * GPT + lane / NL] = szw;
  }
}

// Running "worst candidate" of a thread: smallest accumulated score, latest
// position among equal scores (the one a top-H re-select by (acc desc,
// position asc) leaves out).
struct Worst {
  float a = INFINITY;
  int pos = -1, slot = -1;
  __device__ __forceinline__ void consider(float v, int p, int s) {
    if (v < a || (v == a && p > pos)) { a = v; pos = p; slot = s; }
  }
  __device__ __forceinline__ void merge(float oa, int op, int os) {
    if (os >= 0 && (slot < 0 || oa < a || (oa == a && op > pos))) { a = oa; pos = op; slot = os; }
  }
};

// Block-wide (256 threads): pick the worst candidate and quantize its key and
// value rows into low-bit slot len - cap16 of the unit; free16 becomes the
// dropped slot. Each candidate enters w with its token position (len - 1
// for the slot the new token occupies), which the dropped slot's records
// take. v.imp_bits = 16: the rows are the slot's fp16 rows; 8 or 4: the
// importance tier holds codes, and the row quantized is the slot's codes
// rebuilt in fp16, fp16(code * scale + zero) (the product is exact in fp32,
// so the fused multiply-add rounds once, like the sum of the exact product).
template <int IB, int D, int NL>
__device__ __forceinline__ void imp_row16(const H2OView& v, bool is_v, int64_t slot, int lane, float (&x)[8]) {
  constexpr int CBI = D * IB / 8, GPT = D / (8 * NL);
  uint32_t cw[2];
  load_codes8w<IB>((is_v ? v.vimp : v.kimp) + slot * CBI, lane, cw);
  const uint32_t szw = (is_v ? v.vimpsz : v.kimpsz)[slot * GPT + lane / NL];
  const float s = lo_h(szw), z = hi_h(szw);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = h2f(f2h(fmaf(static_cast<float>(code_of<IB>(cw, e)), s, z)));
}

// Per-channel key tiles: the dropped pair goes to buffer row r = (len -
// cap16) mod 64 as fp16; when r is the last row the buffer becomes tile
// (len - cap16) / 64 (keys per channel, values per token, posq from posbuf),
// its last row taken from the importance slot itself.
template <int D, int BITS, int NL>
__device__ __forceinline__ void demote_to_buffer(const H2OView& v, int unit, int drop, int pos) {
  __shared__ uint16_t s_x[kKeyTile * D];
  __shared__ uint8_t s_c[kKeyTile * D];
  constexpr int LPR = D / 8;
  const int tid = threadIdx.x;
  const int D0 = v.len - v.cap16;  // retained tokens before this demotion
  const int r = D0 % kKeyTile, tile = D0 / kKeyTile;
  const int64_t base16 = static_cast<int64_t>(unit) * v.cap16;
  const int64_t bb = static_cast<int64_t>(unit) * kKeyTile;
  const uint16_t* krow = v.k16 + (base16 + drop) * D;
  const uint16_t* vrow = v.v16 + (base16 + drop) * D;
  if (tid < 2 * LPR) {
    const bool is_v = tid >= LPR;
    const int lane = tid % LPR;
    const uint4 x = *reinterpret_cast<const uint4*>((is_v ? vrow : krow) + lane * 8);
    *reinterpret_cast<uint4*>((is_v ? v.vbuf : v.kbuf) + (bb + r) * D + lane * 8) = x;
  }
  if (tid == 0) v.posbuf[bb + r] = pos;
  if (r != kKeyTile - 1) return;  // uniform
  for (int i = tid; i < kKeyTile * LPR; i += 256) {
    const int t = i / LPR, lane = i % LPR;
    const uint16_t* src = (t < kKeyTile - 1) ? v.kbuf + (bb + t) * D : krow;
    *reinterpret_cast<uint4*>(s_x + t * D + lane * 8) = *reinterpret_cast<const uint4*>(src + lane * 8);
  }
  __syncthreads();
  constexpr int CB = D * BITS / 8, GPT = D / (8 * NL);
  const int64_t q0 = static_cast<int64_t>(unit) * v.capq + static_cast<int64_t>(tile) * kKeyTile;
  quantize_key_tile<D, BITS>(s_x, s_c, v.kq + q0 * CB,
                             v.kcsz + (static_cast<int64_t>(unit) * (v.capq / kKeyTile) + tile) * D);
  quantize_value_tile<D, BITS, NL>(v.vbuf + bb * D, vrow, v.vq + q0 * CB, v.vsz + q0 * GPT);
  for (int t = tid; t < kKeyTile; t += 256) v.posq[q0 + t] = (t < kKeyTile - 1) ? v.posbuf[bb + t] : pos;
}

template <int D, int BITS, int NL, bool KT = false>
__device__ void h2o_select_demote(Worst w, const H2OView& v, int unit) {
  __shared__ float s_acc[4];
  __shared__ int s_pos[4];
  __shared__ int s_slot[4];
  __shared__ int s_drop, s_dpos;
  const int tid = threadIdx.x;
  // wave argmin: within each row by DPP (quad swaps, then the half-row and
  // row mirrors), across rows by the permlane swaps; merge keeps the minimum
  // of a total order, so each pair combines in either order
  w.merge(dpp<0xB1>(w.a), dppi<0xB1>(w.pos), dppi<0xB1>(w.slot));
  w.merge(dpp<0x4E>(w.a), dppi<0x4E>(w.pos), dppi<0x4E>(w.slot));
  w.merge(dpp<0x141>(w.a), dppi<0x141>(w.pos), dppi<0x141>(w.slot));
  w.merge(dpp<0x140>(w.a), dppi<0x140>(w.pos), dppi<0x140>(w.slot));
  {
    const LanePair a = pair_xor32(f2u(w.a)), p = pair_xor32(static_cast<uint32_t>(w.pos)),
                   s = pair_xor32(static_cast<uint32_t>(w.slot));
    Worst x;
    x.merge(u2f(a.a), static_cast<int>(p.a), static_cast<int>(s.a));
    x.merge(u2f(a.b), static_cast<int>(p.b), static_cast<int>(s.b));
    w = x;
  }
  {
    const LanePair a = pair_xor16(f2u(w.a)), p = pair_xor16(static_cast<uint32_t>(w.pos)),
                   s = pair_xor16(static_cast<uint32_t>(w.slot));
    Worst x;
    x.merge(u2f(a.a), static_cast<int>(p.a), static_cast<int>(s.a));
    x.merge(u2f(a.b), static_cast<int>(p.b), static_cast<int>(s.b));
    w = x;
  }
  if (tid % kWave == 0) { s_acc[tid / kWave] = w.a; s_pos[tid / kWave] = w.pos; s_slot[tid / kWave] = w.slot; }
  __syncthreads();
  if (tid == 0) {
    Worst b;
    b.a = s_acc[0]; b.pos = s_pos[0]; b.slot = s_slot[0];
    for (int i = 1; i < 4; ++i) b.merge(s_acc[i], s_pos[i], s_slot[i]);
    s_drop = b.slot;
    s_dpos = b.pos;
  }
  __syncthreads();
  const int drop = s_drop;
  if (drop < 0) return;  // unreachable when heavy + recent == cap16 - 1
  // the dropped token's position, as the candidates were ranked with it (the
  // new token's, len - 1, for the free slot): no second read of pos16
  const int pos = s_dpos;
  if constexpr (KT) {
    if (tid == 0) {
      v.free16[unit] = drop;
      if (v.demoted_pos) v.demoted_pos[unit] = pos;
    }
    demote_to_buffer<D, BITS, NL>(v, unit, drop, pos);
    return;
  }
  constexpr int LPR = D / 8;
  constexpr int CB = D * BITS / 8;
  constexpr int GPT = D / (8 * NL);
  const int64_t base16 = static_cast<int64_t>(unit) * v.cap16;
  const int64_t qslot = static_cast<int64_t>(unit) * v.capq + (v.len - v.cap16);
  // threads [0, LPR) quantize the key row, [LPR, 2*LPR) the value row
  if (tid < 2 * LPR) {
    const int lane = tid % LPR;
    const bool is_v = tid >= LPR;
    float x[8];
    if (v.imp_bits == 16) {
      const uint16_t* src = (is_v ? v.v16 : v.k16) + (base16 + drop) * D + lane * 8;
      load8(src, x);
    } else if (v.imp_bits == 8) {
      imp_row16<8, D, NL>(v, is_v, base16 + drop, lane, x);
    } else {
      imp_row16<4, D, NL>(v, is_v, base16 + drop, lane, x);
    }
    uint32_t szw;
    const uint32_t packed = quantize8<BITS, NL>(x, &szw);
    store_codes8<BITS>((is_v ? v.vq : v.kq) + qslot * CB, lane, packed);
    if (lane % NL == 0) (is_v ? v.vsz : v.ksz)[qslot * GPT + lane / NL] = szw;
  }
  if (tid == 0) {
    v.posq[qslot] = pos;
    v.free16[unit] = drop;
    if (v.demoted_pos) v.demoted_pos[unit] = pos;
  }
}

}  // namespace mikv
