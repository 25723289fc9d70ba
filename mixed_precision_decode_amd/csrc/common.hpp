// Shared device helpers of the MiKV HIP library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mikv {

constexpr int kWave = 64;

__device__ __forceinline__ float h2f(uint16_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, bits));
}
// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint16_t f2h(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
// fp32 product rounded to fp32 before anything else: the empty asm keeps the
// compiler from fusing the multiply with a following fp16 conversion
// (v_fma_mixlo_f16 rounds once), so fp16(mul_rn(a, b)) is the two-step
// rounding fp16(fp32(a*b)).
__device__ __forceinline__ float mul_rn(float a, float b) {
  float p = a * b;
  asm volatile("" : "+v"(p));
  return p;
}
__device__ __forceinline__ float lo_h(uint32_t w) { return h2f(static_cast<uint16_t>(w & 0xFFFFu)); }
__device__ __forceinline__ float hi_h(uint32_t w) { return h2f(static_cast<uint16_t>(w >> 16)); }

// ---------------------------------------------------------------------------
// Cross-lane data movement inside a row of 16 lanes (DPP) and across rows.
// DPP controls: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140, row_ror:n = 0x120 + n.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

// Sum / max over aligned groups of N lanes (N in {1,2,4,8,16}); every lane of
// the group ends with the result.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<0xB1>(v);
  if constexpr (N >= 4) v += dpp<0x4E>(v);
  if constexpr (N >= 8) v += dpp<0x141>(v);
  if constexpr (N >= 16) v += dpp<0x140>(v);
  return v;
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp<0xB1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp<0x4E>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp<0x141>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp<0x140>(v));
  return v;
}
template <int N>
__device__ __forceinline__ float group_min(float v) {
  if constexpr (N >= 2) v = fminf(v, dpp<0xB1>(v));
  if constexpr (N >= 4) v = fminf(v, dpp<0x4E>(v));
  if constexpr (N >= 8) v = fminf(v, dpp<0x141>(v));
  if constexpr (N >= 16) v = fminf(v, dpp<0x140>(v));
  return v;
}

// Cross-row steps of a wave reduction on gfx950 (v_permlane32_swap,
// v_permlane16_swap: vector ALU, no LDS). The pair holds, in some order, the
// values of lanes l and l ^ 32 (l ^ 16), so a commutative combine of its two
// halves needs no per-row select and every lane ends with the same result.
struct LanePair { uint32_t a, b; };
__device__ __forceinline__ LanePair pair_xor32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return {static_cast<uint32_t>(r[0]), static_cast<uint32_t>(r[1])};
}
__device__ __forceinline__ LanePair pair_xor16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return {static_cast<uint32_t>(r[0]), static_cast<uint32_t>(r[1])};
}
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// Sum / max over the wave's four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float rows_sum(float v) {
  LanePair x = pair_xor32(f2u(v));
  v = u2f(x.a) + u2f(x.b);
  x = pair_xor16(f2u(v));
  return u2f(x.a) + u2f(x.b);
}
__device__ __forceinline__ float rows_max(float v) {
  LanePair x = pair_xor32(f2u(v));
  v = fmaxf(u2f(x.a), u2f(x.b));
  x = pair_xor16(f2u(v));
  return fmaxf(u2f(x.a), u2f(x.b));
}

// DPP move of v under control CTRL into the rows set in ROWMASK; other rows,
// and lanes whose source is out of the row when BC is set, read 0.
template <int CTRL, int ROWMASK, bool BC>
__device__ __forceinline__ int dpp_rows(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xF, BC); }

// Inclusive prefix sum of an int over the wave's 64 lanes (all active): a
// Hillis-Steele scan inside each 16-lane row (DPP row_shr 1, 2, 4, 8, lanes
// before the row start reading 0), then row_bcast:15 adds the end of rows 0
// and 2 to rows 1 and 3, and row_bcast:31 the end of row 1 to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_rows<0x111, 0xF, true>(v);
  v += dpp_rows<0x112, 0xF, true>(v);
  v += dpp_rows<0x114, 0xF, true>(v);
  v += dpp_rows<0x118, 0xF, true>(v);
  v += dpp_rows<0x142, 0xA, false>(v);
  v += dpp_rows<0x143, 0xC, false>(v);
  return v;
}

// Sum / max over the whole wave (all 64 lanes active); every lane ends with
// the result.
__device__ __forceinline__ float wave_sum(float v) { return rows_sum(group_sum<16>(v)); }
__device__ __forceinline__ float wave_max(float v) { return rows_max(group_max<16>(v)); }

// ---------------------------------------------------------------------------
// Per-token asymmetric quantization of one group held by NL lanes, 8
// channels per lane (velog notes "No Token Left Behind ...", Key
// contributions 1) and 2): per-token asymmetric codes, groups of d/2).
// Fixed fp32 sequence: scale = fp16((max - min) / qmax), zero = min,
// code = clamp(rint((x - zero) / scale), 0, qmax); zeros stored as +0.
// Returns the packed codes of the lane's 8 channels in the low 8*BITS bits
// and writes (scale | zero << 16) to *sz_word.
// ---------------------------------------------------------------------------
template <int BITS, int NL>
__device__ __forceinline__ void quantize8_values(const float (&x)[8], uint32_t* sz_word, float (&t)[8]) {
  constexpr float qmax = static_cast<float>((1 << BITS) - 1);
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  mn = group_min<NL>(mn);
  mx = group_max<NL>(mx);
  const float s32 = (mx - mn) / qmax;
  uint16_t s16 = f2h(s32);
  if ((s16 & 0x7FFFu) == 0) s16 = 0;
  uint16_t z16 = f2h(mn);  // exact: mn is an fp16 value
  if ((z16 & 0x7FFFu) == 0) z16 = 0;
  *sz_word = static_cast<uint32_t>(s16) | (static_cast<uint32_t>(z16) << 16);
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = 0.0f;
  if (s16 != 0) {
    const float s = h2f(s16);
    const float z = h2f(z16);
    // code = rint of the IEEE quotient fl((x - z) / s), found without the
    // divide: y = (x - z) * rcp(s) is within 1.6 * 2^-23 |Q| of the exact
    // quotient Q (rcp within 1 ulp, one rounded multiply) and fl(Q) within
    // 2^-24 |Q|, so |y - fl(Q)| <= 2^-22 |Q|: 2^-18 for the 2- and 4-bit
    // codes' range |Q| <= 16, 2^-14 for 8-bit codes (|Q| <= 256).
    // When y is farther than the margin (2^-16, or 2^-13 at 8 bits) from its
    // nearest half-integer, y and fl(Q) lie in the same rounding interval
    // and rint(y) = rint(fl(Q)). The distance is taken as |fma(x - z, r,
    // -rint(y))|, the exact product's distance from rint(y) rounded once: it
    // differs from |y - rint(y)| by at most half an ulp of y (2^-20 at
    // |y| <= 16, 2^-16 at |y| <= 256), which the margins leave room for. A
    // lane whose largest distance reaches 1/2 - margin (about 1e-5 of
    // values, 1e-4 at 8 bits) takes the IEEE divide for all its values.
    constexpr float kFar = 0.5f - (BITS == 8 ? 0x1p-13f : 0x1p-16f);
    const float r = __builtin_amdgcn_rcpf(s);
    float dist = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = x[i] - z;  // exact: fp16 values
      t[i] = rintf(a * r);
      dist = fmaxf(dist, fabsf(fmaf(a, r, -t[i])));
    }
    if (dist >= kFar) {
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = rintf((x[i] - z) / s);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = __builtin_amdgcn_fmed3f(t[i], 0.0f, qmax);
  }
}

template <int BITS, int NL>
__device__ __forceinline__ void quantize8_codes(const float (&x)[8], uint32_t* sz_word, uint32_t (&code)[8]) {
  float t[8];
  quantize8_values<BITS, NL>(x, sz_word, t);
#pragma unroll
  for (int i = 0; i < 8; ++i) code[i] = static_cast<uint32_t>(t[i]);
}

// Packed codes of the lane's 8 channels (BITS <= 4: the low 8*BITS bits).
// Each code goes into a byte with one v_cvt_pk_u8_f32; the bytes are then
// merged: INT4 even channels' bytes | odd channels' bytes << 4; INT2 four
// words of two bytes (channels m and 4 + m) shifted by 2m.
template <int BITS, int NL>
__device__ __forceinline__ uint32_t quantize8(const float (&x)[8], uint32_t* sz_word) {
  static_assert(BITS == 4 || BITS == 2, "4- or 2-bit codes");
  float t[8];
  quantize8_values<BITS, NL>(x, sz_word, t);
  if constexpr (BITS == 4) {
    uint32_t a = 0u, b = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a = __builtin_amdgcn_cvt_pk_u8_f32(t[2 * k], k, a);
      b = __builtin_amdgcn_cvt_pk_u8_f32(t[2 * k + 1], k, b);
    }
    return a | (b << 4);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      w[m] = __builtin_amdgcn_cvt_pk_u8_f32(t[m], 0, 0u);
      w[m] = __builtin_amdgcn_cvt_pk_u8_f32(t[4 + m], 1, w[m]);
    }
    return w[0] | (w[1] << 2) | (w[2] << 4) | (w[3] << 6);
  }
}

// The 8 codes packed at QB bits (8, 4 or 2) into w[0..1]: byte j of the
// 8-bit form holds channel j; the 4- and 2-bit forms use w[0] only.
template <int QB>
__device__ __forceinline__ void pack8(const uint32_t (&code)[8], uint32_t (&w)[2]) {
  if constexpr (QB == 8) {
    w[0] = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
    w[1] = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
  } else {
    w[0] = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w[0] |= code[i] << (QB * i);
    w[1] = 0;
  }
}

// Code of channel e (0..7) of a lane's QB-bit codes w[0..1].
template <int QB>
__device__ __forceinline__ uint32_t code_of(const uint32_t* w, int e) {
  if constexpr (QB == 8) return (w[e / 4] >> (8 * (e % 4))) & 0xFFu;
  else return (w[0] >> (QB * e)) & ((1u << QB) - 1u);
}

// Streaming loads with the nontemporal hint (the cache rows of a decode
// step are read once; the hint keeps them from displacing reused lines).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint2 ld_nt8(const void* p) {
  const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(t.x, t.y);
}
__device__ __forceinline__ uint32_t ld_nt4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// Load 8 fp16 values (16 bytes) and widen to fp32.
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  x[0] = lo_h(w.x); x[1] = hi_h(w.x);
  x[2] = lo_h(w.y); x[3] = hi_h(w.y);
  x[4] = lo_h(w.z); x[5] = hi_h(w.z);
  x[6] = lo_h(w.w); x[7] = hi_h(w.w);
}

// Store packed codes of 8 channels: INT8 -> 8 bytes, INT4 -> one 32-bit
// word, INT2 -> 16 bits.
template <int BITS>
__device__ __forceinline__ void store_codes8w(uint8_t* row_codes, int lane_in_row, const uint32_t (&w)[2]) {
  if constexpr (BITS == 8) {
    reinterpret_cast<uint2*>(row_codes)[lane_in_row] = make_uint2(w[0], w[1]);
  } else if constexpr (BITS == 4) {
    reinterpret_cast<uint32_t*>(row_codes)[lane_in_row] = w[0];
  } else {
    reinterpret_cast<uint16_t*>(row_codes)[lane_in_row] = static_cast<uint16_t>(w[0]);
  }
}
// Load the packed codes of a lane's 8 channels (the inverse of store_codes8w).
template <int BITS>
__device__ __forceinline__ void load_codes8w(const uint8_t* row_codes, int lane_in_row, uint32_t (&w)[2]) {
  if constexpr (BITS == 8) {
    const uint2 t = reinterpret_cast<const uint2*>(row_codes)[lane_in_row];
    w[0] = t.x; w[1] = t.y;
  } else if constexpr (BITS == 4) {
    w[0] = reinterpret_cast<const uint32_t*>(row_codes)[lane_in_row];
    w[1] = 0;
  } else {
    w[0] = reinterpret_cast<const uint16_t*>(row_codes)[lane_in_row];
    w[1] = 0;
  }
}

// Store packed codes of 8 channels: INT4 -> one 32-bit word, INT2 -> 16 bits.
template <int BITS>
__device__ __forceinline__ void store_codes8(uint8_t* row_codes, int lane_in_row, uint32_t packed) {
  if constexpr (BITS == 4) {
    reinterpret_cast<uint32_t*>(row_codes)[lane_in_row] = packed;
  } else {
    reinterpret_cast<uint16_t*>(row_codes)[lane_in_row] = static_cast<uint16_t>(packed);
  }
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 is treated as +0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace mikv
