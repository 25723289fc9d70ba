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
  uint16_t* k16;
  uint16_t* v16;
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
// len - 1).
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
    const uint16_t* src = (is_v ? v.v16 : v.k16) + (base16 + drop) * D + lane * 8;
    float x[8];
    load8(src, x);
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
