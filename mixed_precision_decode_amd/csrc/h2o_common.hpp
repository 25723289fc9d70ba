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
};

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
// dropped slot. `fr` is the slot the new token occupies (its position is
// len - 1). v.imp_bits = 16: the rows are the slot's fp16 rows; 8 or 4: the
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

template <int D, int BITS, int NL>
__device__ void h2o_select_demote(Worst w, const H2OView& v, int unit, int fr) {
  __shared__ float s_acc[4];
  __shared__ int s_pos[4];
  __shared__ int s_slot[4];
  __shared__ int s_drop;
  const int tid = threadIdx.x;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float oa = shfl_xor_f(w.a, m);
    const int op = __shfl_xor(w.pos, m);
    const int os = __shfl_xor(w.slot, m);
    w.merge(oa, op, os);
  }
  if (tid % kWave == 0) { s_acc[tid / kWave] = w.a; s_pos[tid / kWave] = w.pos; s_slot[tid / kWave] = w.slot; }
  __syncthreads();
  if (tid == 0) {
    Worst b;
    b.a = s_acc[0]; b.pos = s_pos[0]; b.slot = s_slot[0];
    for (int i = 1; i < 4; ++i) b.merge(s_acc[i], s_pos[i], s_slot[i]);
    s_drop = b.slot;
  }
  __syncthreads();
  const int drop = s_drop;
  if (drop < 0) return;  // unreachable when heavy + recent == cap16 - 1
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
    const int pos = (drop == fr) ? v.len - 1 : v.pos16[base16 + drop];
    v.posq[qslot] = pos;
    v.free16[unit] = drop;
    if (v.demoted_pos) v.demoted_pos[unit] = pos;
  }
}

}  // namespace mikv
