// Head tiles (2-4 query heads sharing a kv head) of the split kernel, with the
// key scores on the matrix cores.
//
// velog notes "No Token Left Behind ...", section 3.4: decode attention is a
// batched matrix-vector product over a precision-grouped cache. With g query
// heads per kv head the product against the keys is a small matrix product
// (heads x tokens x channels); here it runs as v_mfma_f32_16x16x32_f16:
//   A = q-hat, head h in row 4h (the other rows zero), k = 32 channels;
//   B = keys of 16 tokens, k = the same 32 channels, columns = tokens;
//   D = scores: register 0 of lane 16h + t holds head h's score of token t,
//   so with 4 heads each lane of the wave carries one (token, head) score.
// q-hat enters as two fp16 operands, hi = fp16(q-hat) and lo = fp16(q-hat -
// hi), accumulated into the same D, so the product keeps about 22 bits of
// q-hat (fp32 q-hat is the reading the method needs: the query stays floating
// point). Low-bit key codes enter as the exact fp16 values 1 + code * step
// (tile_codes; the matrix cores do not take fp16 subnormal operands exactly,
// so the code cannot simply sit in the low mantissa bits). Per group of d/2
// channels the product is then sum(q) + step * (q . code), where sum(q) is
// what the matrix cores form against B = 1 (taken once, at the start). The
// score of a low-bit token, scale * (q . code) + zero * sum(q), becomes
// (scale / step) * product + (zero - scale / step) * sum(q): two per-token
// coefficients, so the channels of one MFMA never span two groups.
//
// Every (token, head) score, its exp and its running-max check are computed
// once, on the lane that holds it. The value sums stay on the vector ALUs in
// row layout (8 channels per lane, the token's probability times the value
// scale read from LDS); the zero-point part sum(p * zero) is kept per head and
// group on the score lanes. The running maximum per head is lazy: it moves
// only when a score exceeds it by more than kTileHeadroom (log2 units), so
// the rescaling of the sums is rare and the common path has no reduction.
//
// The importance tier is either fp16 rows (QB = 16) or, for a reduced-
// precision importance cache (velog notes, Key contributions 3); paperlayer
// summary, section 3.3), codes of 8 or 4 bits read exactly like the retained
// tier's; the new token is then quantized as it is appended and enters the
// attention through its dequantized codes.
#pragma once

#ifndef MIKV_TILE_NS
#define MIKV_TILE_NS 2
#endif

typedef _Float16 tile_h8 __attribute__((ext_vector_type(8)));
typedef float tile_f4 __attribute__((ext_vector_type(4)));
typedef unsigned int tile_u4 __attribute__((ext_vector_type(4)));

constexpr float kTileHeadroom = 16.0f;
constexpr int kTileG = 16;  // tokens per MFMA group
constexpr float kTileCodeUnit = 0x1p24f;  // value codes sum as fp16 subnormals, code * 2^-24

// Value codes enter the value sums as fp16 subnormals: a code masked in
// place inside a 16-bit half, so each half reads as code * 2^(p - 24) for the
// code's bit position p (p + bits <= 10 keeps the exponent field zero). One
// AND gives the codes of two channels (two tokens for 2-bit codes). The
// factor that turns channel e's sum back into code units:
//   4-bit (channel c at bits 4c of a token's word): even channels sit at bit
//     0 of a half, odd ones at bit 4;
//   2-bit (channel c at bits 2c of a token's 16 bits): channels 0..4 at bits
//     2c, channels 5..7, shifted down by 10, at bits 2(c - 5);
//   8-bit: every code at bit 0.
template <int QB>
__device__ __forceinline__ constexpr float tile_val_unit(int e) {
  if constexpr (QB == 4) return (e % 2) ? 0x1p20f : 0x1p24f;
  else if constexpr (QB == 2) return 0x1p24f / static_cast<float>(1 << (2 * (e < 5 ? e : e - 5)));
  else return kTileCodeUnit;
}

// Element e of chunk c (32 channels) for lane group r: the channel it holds.
// Chunks 0..CPG-1 cover group 0 (channels [0, d/2)), the rest group 1; lane
// group r takes a contiguous run of 8*CPG channels of each group. Within the
// 8 channels of a chunk the order is the one the code conversion produces.
template <int D, int QB>
__device__ __forceinline__ constexpr int tile_chan(int c, int r, int e) {
  constexpr int CPG = D / 64, G = D / 2;
  int pe = e;
  if constexpr (QB == 4) pe = (e < 4) ? 2 * e : 2 * (e - 4) + 1;
  if constexpr (QB == 2) pe = (e % 2 == 0) ? e / 2 : 4 + e / 2;
  return (c / CPG) * G + 8 * CPG * r + (c % CPG) * 8 + pe;
}

// Sum over the lanes of the wave that share lane % S (S in {8, 16}).
template <int S>
__device__ __forceinline__ float slot_sum(float v) {
  static_assert(S == 8 || S == 16, "value slices of 8 channels: 8 or 16 lanes per row");
  if constexpr (S == 8) v += dpp<0x128>(v);  // row_ror:8 -> lane ^ 8 within the row
  return rows_sum(v);
}

template <int NB>
struct TileBytes { uint32_t w[(NB + 3) / 4]; };

// NB bytes at byte offset off of a buffer resource (NB in {2, 4, 8, 16, 32}).
template <int NB>
__device__ __forceinline__ void tile_load(Rsrc r, uint32_t off, uint32_t* w) {
  if constexpr (NB == 32) {
    const Words<4> a = bload<4>(r, off), b = bload<4>(r, off + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) { w[i] = a.w[i]; w[4 + i] = b.w[i]; }
  } else if constexpr (NB == 16) {
    const Words<4> a = bload<4>(r, off);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = a.w[i];
  } else if constexpr (NB == 8) {
    const Words<2> a = bload<2>(r, off);
    w[0] = a.w[0]; w[1] = a.w[1];
  } else if constexpr (NB == 4) {
    w[0] = bload1(r, off);
  } else {
    w[0] = static_cast<uint32_t>(
        __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, kBufNT));
  }
}

// Codes as matrix-core operands. 2- and 4-bit codes become the exact fp16
// values 1 + code * kCodeStep: the code goes to the top of the mantissa under
// the exponent of 1.0 (2-bit: bits 8-9, a byte 0x3C | code over a zero byte;
// 4-bit: bits 4-7, the nibble over a 0x3C byte), so building an operand takes
// byte moves and masks only, and a product with it is sum(A) + step * (A .
// code), sum(A) being taken back out by the caller. 8-bit codes fill the
// whole low mantissa byte under 1024 (magic byte 0x64) and one packed
// subtraction per operand gives the integers.
template <int QB>
constexpr float kCodeStep = QB == 2 ? 0.25f : (QB == 4 ? 0x1p-6f : 1.0f);
template <int QB>
constexpr uint32_t kCodeMagic = QB == 8 ? 0x64646464u : 0x3C3C3C3Cu;

// The 8 codes of part `part` of a lane's group words -> the MFMA operand
// (order of tile_chan); magic = kCodeMagic<QB>, kept in a register.
template <int QB>
__device__ __forceinline__ tile_h8 tile_codes(const uint32_t* w, int part, uint32_t magic) {
  constexpr uint32_t kLo = 0x04010400u, kHi = 0x04030402u;
  tile_u4 u;
  if constexpr (QB == 8) {  // 8 bytes in two words, channel order kept
    const uint32_t a = w[2 * part], b = w[2 * part + 1];
    u[0] = __builtin_amdgcn_perm(magic, a, kLo);
    u[1] = __builtin_amdgcn_perm(magic, a, kHi);
    u[2] = __builtin_amdgcn_perm(magic, b, kLo);
    u[3] = __builtin_amdgcn_perm(magic, b, kHi);
    return __builtin_bit_cast(tile_h8, u) - static_cast<tile_h8>(static_cast<_Float16>(1024.0f));
  } else if constexpr (QB == 4) {  // 8 nibbles of one word, each moved to the top of its byte
    const uint32_t x = w[part];
    const uint32_t lo = (x << 4) & 0xF0F0F0F0u, hi = x & 0xF0F0F0F0u;
    u[0] = __builtin_amdgcn_perm(magic, lo, kLo);
    u[1] = __builtin_amdgcn_perm(magic, lo, kHi);
    u[2] = __builtin_amdgcn_perm(magic, hi, kLo);
    u[3] = __builtin_amdgcn_perm(magic, hi, kHi);
  } else {  // 8 crumbs in half `part` of the word: crumb m of its two bytes
    // as 0x3C | code (one v_and_or_b32, magic in a register), each over a
    // zero byte: [0, y.b(2 part), 0, y.b(2 part + 1)]
    const uint32_t x = w[0];
    const uint32_t sel = part ? 0x03040204u : 0x01040004u;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t y = ((x >> (2 * m)) & 0x03030303u) | magic;
      u[m] = __builtin_amdgcn_perm(0u, y, sel);
    }
  }
  return __builtin_bit_cast(tile_h8, u);
}

// Per-head sums of q-hat over the two channel groups as the matrix cores
// form them (B = 1; the result's lane 0 holds rows 0..3 = the heads), made
// wave-uniform.
template <int NCH, int RT>
__device__ __forceinline__ void tile_qsums(const tile_h8 (&qa_hi)[NCH], const tile_h8 (&qa_lo)[NCH],
                                           float (&qs)[RT][2]) {
  constexpr int CPG = NCH / 2;
  const tile_h8 ones = static_cast<tile_h8>(static_cast<_Float16>(1.0f));
  tile_f4 s[2];
  s[0] = tile_f4{0.0f, 0.0f, 0.0f, 0.0f};
  s[1] = s[0];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    s[c / CPG] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[c], ones, s[c / CPG], 0, 0, 0);
    s[c / CPG] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_lo[c], ones, s[c / CPG], 0, 0, 0);
  }
#pragma unroll
  for (int gi = 0; gi < 2; ++gi)
#pragma unroll
    for (int h = 0; h < RT; ++h) {
      // copied to a scalar first: __builtin_bit_cast of a vector element
      // compiles into element 0 whatever the index
      const float v = s[gi][h];
      qs[h][gi] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    }
}

// The same sums with head h in A row 4h (tile_split's layout): D row 4h is
// register 0 of lane group h, so each lane gets the sums of its own head
// (zero on lane groups >= RT).
template <int NCH>
__device__ __forceinline__ void tile_qsums_lane(const tile_h8 (&qa_hi)[NCH], const tile_h8 (&qa_lo)[NCH],
                                                float (&qs)[2]) {
  constexpr int CPG = NCH / 2;
  const tile_h8 ones = static_cast<tile_h8>(static_cast<_Float16>(1.0f));
  tile_f4 s[2];
  s[0] = tile_f4{0.0f, 0.0f, 0.0f, 0.0f};
  s[1] = s[0];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    s[c / CPG] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[c], ones, s[c / CPG], 0, 0, 0);
    s[c / CPG] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_lo[c], ones, s[c / CPG], 0, 0, 0);
  }
  qs[0] = s[0][0];
  qs[1] = s[1][0];
}

// A-operand row ai of the tile's query heads: head ai (rows RT..15 zero),
// or with SPREAD head ai / 4 in rows 0, 4, 8, 12 (the others zero), which
// puts head h's scores in register 0 of lane group h. -1: a zero row.
template <int RT, bool SPREAD>
__device__ __forceinline__ int tile_row_head(int ai) {
  if constexpr (SPREAD) return (ai % 4 == 0 && ai / 4 < RT) ? ai / 4 : -1;
  else return ai < RT ? ai : -1;
}

// q and b of the tile's A operand: lane (row ai, lane group ar) takes the
// 8-channel runs tile_chan<D, 16>(c, ar, 0) of the query head of row ai.
// Only lanes of live rows fetch: the others read at the end of the
// buffers, which a raw buffer load returns as zeros without a memory access
// (their q-hat is set to 0 afterwards). Every block of the kv head reads the
// same q and b, so these loads keep the default cache policy.
template <int D, int RT, bool SPREAD = false>
__device__ __forceinline__ void tile_load_qb(const DecodeK& p, int n, int g, int tile, const float* bvec, int ai,
                                             int ar, float (&qv)[D / 32][8], float (&bv)[D / 32][8]) {
  const Rsrc rq = make_rsrc(p.q + (static_cast<int64_t>(n) * p.hq + g * p.rep + tile * RT) * D, RT * D * 2);
  const Rsrc rb = make_rsrc(bvec, D * 4);
  const int hr = tile_row_head<RT, SPREAD>(ai);
  const bool live = hr >= 0;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const int base = tile_chan<D, 16>(c, ar, 0);
    const auto qw = __builtin_amdgcn_raw_buffer_load_b128(rq, live ? (hr * D + base) * 2 : RT * D * 2, 0, 0);
    const auto b0 = __builtin_amdgcn_raw_buffer_load_b128(rb, live ? base * 4 : D * 4, 0, 0);
    const auto b1 = __builtin_amdgcn_raw_buffer_load_b128(rb, live ? base * 4 + 16 : D * 4, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[c][2 * i] = lo_h(qw[i]);
      qv[c][2 * i + 1] = hi_h(qw[i]);
      bv[c][i] = u2f(b0[i]);
      bv[c][4 + i] = u2f(b1[i]);
    }
  }
}

template <int D, int QB>
struct TileRegs {
  static constexpr int CPG = D / 64;
  static constexpr int KB = CPG * 8 * QB / 8;                 // key bytes per lane and group
  static constexpr int KW = (KB + 3) / 4;                     // words per lane and group
  static constexpr int LPTV = D / 8, VSLOTS = 64 / LPTV, VTPL = kTileG / VSLOTS;
  static constexpr int VB = QB;                               // value bytes per lane and token (8 channels)
  static constexpr int VW = (VB + 3) / 4;
  uint32_t k[2][KW];
  uint32_t ksz[2], vsz[2];
  uint32_t v[VTPL][VW];
};

// QB: bits per value of this tier (16 = fp16 rows); IMPT: the importance
// tier (free slot, scores for p16, the new token) rather than the retained.
template <int D, int QB, int RT, bool IMPT>
__device__ __forceinline__ void tile_split(const DecodeK& p, int unit, int n, int g, int tile, int split,
                                           const float* bvec, float* red, float (*sm)[RT], float* po,
                                           float2* pml, float (*wbuf)[kTileG][2][RT]) {
  using R_t = TileRegs<D, QB>;
  constexpr bool F16T = QB == 16;
  constexpr int NCH = D / 32, CPG = D / 64, G = D / 2;
  constexpr int LPTV = R_t::LPTV, VSLOTS = R_t::VSLOTS, VTPL = R_t::VTPL;
  constexpr int ROWB = D * QB / 8;  // bytes per token row
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int ai = lane % 16, ar = lane / 16;           // MFMA row / k block of this lane
  const int vs = lane / LPTV, vj = lane % LPTV;       // value slot, 8-channel slice
  const int vg = (8 * vj) / G;                        // value group of the slice

  // ---- block range and buffer resources
  int nt, frel = -1;
  Rsrc rk, rv, rks, rvs;
  int64_t scb = 0, rb16 = 0;
  if constexpr (IMPT) {
    const int s0 = split * p.C16;
    const int s1 = min(p.cap16, s0 + p.C16);
    nt = max(s1 - s0, 0);
    rb16 = static_cast<int64_t>(unit) * p.cap16;
    frel = p.free16[unit] - s0;
    if constexpr (F16T) {
      rk = make_rsrc(p.k16 + (rb16 + s0) * D, static_cast<uint32_t>(nt) * ROWB);
      rv = make_rsrc(p.v16 + (rb16 + s0) * D, static_cast<uint32_t>(nt) * ROWB);
      rks = rk;  // no scales on an fp16 tier
      rvs = rv;
    } else {
      rk = make_rsrc(p.kimp + (rb16 + s0) * ROWB, static_cast<uint32_t>(nt) * ROWB);
      rv = make_rsrc(p.vimp + (rb16 + s0) * ROWB, static_cast<uint32_t>(nt) * ROWB);
      rks = make_rsrc(p.kimpsz + (rb16 + s0) * 2, static_cast<uint32_t>(nt) * 8);
      rvs = make_rsrc(p.vimpsz + (rb16 + s0) * 2, static_cast<uint32_t>(nt) * 8);
    }
    scb = (static_cast<int64_t>(unit) * p.rep + tile * RT) * p.cap16 + s0;
  } else {
    const int t0 = (split - p.S16) * p.Cq;
    const int t1 = min(p.nq, t0 + p.Cq);
    nt = max(t1 - t0, 0);
    const int64_t ub = static_cast<int64_t>(unit) * p.capq + t0;
    rk = make_rsrc(p.kq + ub * ROWB, static_cast<uint32_t>(nt) * ROWB);
    rv = make_rsrc(p.vq + ub * ROWB, static_cast<uint32_t>(nt) * ROWB);
    rks = make_rsrc(p.ksz + ub * 2, static_cast<uint32_t>(nt) * 8);
    rvs = make_rsrc(p.vsz + ub * 2, static_cast<uint32_t>(nt) * 8);
  }

  auto load = [&](int grp, R_t& R) {
    const uint32_t tb = static_cast<uint32_t>(grp * kTileG);
    const uint32_t tk = tb + ai;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const uint32_t ch0 = gi * G + 8 * CPG * ar;
      tile_load<R_t::KB>(rk, tk * ROWB + ch0 * QB / 8, R.k[gi]);
    }
    if constexpr (!F16T) {
      const Words<2> ks = bload<2>(rks, tk * 8), vz = bload<2>(rvs, tk * 8);
      R.ksz[0] = ks.w[0]; R.ksz[1] = ks.w[1];
      R.vsz[0] = vz.w[0]; R.vsz[1] = vz.w[1];
    }
#pragma unroll
    for (int k = 0; k < VTPL; ++k) {
      const uint32_t tv = tb + vs + k * VSLOTS;
      tile_load<R_t::VB>(rv, tv * ROWB + vj * R_t::VB, R.v[k]);
    }
  };
  // ---- q and b first, every lane (rows >= RT read zeros and are zeroed
  // below): their wait then covers neither the first groups' loads issued
  // after them nor a branch per chunk
  const float qscale = kLog2e / sqrtf(static_cast<float>(D));
  float qv[NCH][8], bv[NCH][8];
  tile_load_qb<D, RT, true>(p, n, g, tile, bvec, ai, ar, qv, bv);

  // register sets in a ring: NS - 1 groups' loads in flight while one group
  // is computed (two sets; three or four on the low-bit tier measured no
  // faster: the loop is bound by VALU issue, not by loads in flight)
  constexpr int NS = F16T ? 2 : MIKV_TILE_NS;
  R_t R[NS];
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) load(wave + 4 * i, R[i]);

  // ---- q-hat as MFMA A operands (hi and lo halves), per-group sums of q-hat
  tile_h8 qa_hi[NCH], qa_lo[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int base = tile_chan<D, 16>(c, ar, 0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ch = tile_chan<D, QB>(c, ar, e);
      const float qe = qv[c][ch - base] * __builtin_amdgcn_rcpf(bv[c][ch - base]) * qscale;
      const float q = tile_row_head<RT, true>(ai) >= 0 ? qe : 0.0f;
      const _Float16 hi = static_cast<_Float16>(q);
      qa_hi[c][e] = hi;
      qa_lo[c][e] = static_cast<_Float16>(q - static_cast<float>(hi));
    }
  }
  // head h sits in A row 4h, so lane 16 h + t holds head h's score of token
  // t (register 0 of the accumulators); lane groups >= RT hold none
  const int hl = lane / 16;
  // qs[gi] = sum over group gi's channels of the lane's head's q-hat
  float qs[2] = {0.0f, 0.0f};
  if constexpr (!F16T) tile_qsums_lane<NCH>(qa_hi, qa_lo, qs);

  // ---- online-softmax state of the wave: running maximum, sum and
  // zero-point sums of the lane's head (uniform over its lane group, the
  // sums partial per lane), value sums of every head in row layout
  float M = -INFINITY, l = 0.0f, zz[2] = {0.0f, 0.0f};
  float a[RT][8];
#pragma unroll
  for (int h = 0; h < RT; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) a[h][e] = 0.0f;

  // ---- the new token: appended by the tile-0 block that owns the free
  // slot, and seeded into wave 0's state (max = its score, sum = 1, o = v).
  // A code tier stores it quantized and seeds the state with its codes
  // rebuilt (code * scale + zero), as it will be read from then on.
  if constexpr (IMPT) {
    if (frel >= 0 && frel < nt && wave == 0) {  // uniform
      float x[RT];
#pragma unroll
      for (int h = 0; h < RT; ++h) x[h] = 0.0f;
      if (lane < LPTV) {
        const int c0 = 8 * lane;
        const int64_t nb = static_cast<int64_t>(unit) * D + c0;
        const int64_t fs = rb16 + p.free16[unit];
        // every input of the seed in flight at once
        float kx[8], vx[8], b8[8], qn[RT][8];
        load8(p.k_new + nb, kx);
        load8(p.v_new + nb, vx);
#pragma unroll
        for (int e = 0; e < 8; ++e) b8[e] = bvec[c0 + e];
#pragma unroll
        for (int h = 0; h < RT; ++h)
          load8(p.q + (static_cast<int64_t>(n) * p.hq + g * p.rep + tile * RT + h) * D + c0, qn[h]);
#pragma unroll
        for (int e = 0; e < 8; ++e) kx[e] = h2f(f2h(mul_rn(kx[e], b8[e])));  // fp16(k * b)
        if constexpr (F16T) {
          if (tile == 0) {
            uint32_t kw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              kw[i] = static_cast<uint32_t>(f2h(kx[2 * i])) | (static_cast<uint32_t>(f2h(kx[2 * i + 1])) << 16);
            *reinterpret_cast<uint4*>(p.k16 + fs * D + c0) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
            *reinterpret_cast<uint4*>(p.v16 + fs * D + c0) = *reinterpret_cast<const uint4*>(p.v_new + nb);
          }
        } else {
          constexpr int NL = G / 8;  // lanes per quantization group
          uint32_t kszw, vszw, kc[8], vc[8];
          quantize8_codes<QB, NL>(kx, &kszw, kc);
          quantize8_codes<QB, NL>(vx, &vszw, vc);
          if (tile == 0) {
            uint32_t kw2[2], vw2[2];
            pack8<QB>(kc, kw2);
            pack8<QB>(vc, vw2);
            store_codes8w<QB>(p.kimp + fs * ROWB, lane, kw2);
            store_codes8w<QB>(p.vimp + fs * ROWB, lane, vw2);
            if (lane % NL == 0) {
              p.kimpsz[fs * 2 + lane / NL] = kszw;
              p.vimpsz[fs * 2 + lane / NL] = vszw;
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kx[e] = fmaf(static_cast<float>(kc[e]), lo_h(kszw), hi_h(kszw));
            vx[e] = fmaf(static_cast<float>(vc[e]), lo_h(vszw), hi_h(vszw));
          }
        }
        if (tile == 0 && lane == 0) p.pos16[fs] = p.len - 1;
#pragma unroll
        for (int h = 0; h < RT; ++h) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[h] += qn[h][e] * __builtin_amdgcn_rcpf(b8[e]) * qscale * kx[e];
            a[h][e] = F16T ? vx[e] : vx[e] / tile_val_unit<QB>(e);  // code tiers sum in code units
          }
        }
      }
#pragma unroll
      for (int h = 0; h < RT; ++h) {
        x[h] = group_sum<LPTV>(x[h]);
        const float xu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x[h]), 0));
        if (hl == h) {
          M = xu;
          if (lane % 16 == 0) l = 1.0f;
        }
        if (lane == 0) p.sc16[scb + static_cast<int64_t>(h) * p.cap16 + frel] = xu;
      }
    }
  }

  // key codes as 1 + code * step for the MFMA (tile_codes); value codes as
  // fp16 subnormals (masked in place, or for 8-bit codes a byte under a zero
  // byte), which v_fma_mix takes exactly: the value sums carry no offset to
  // cancel later
  const uint32_t kmagic = opaque(kCodeMagic<QB>), magic = opaque(0u);
  auto step = [&](const R_t& R, int grp) {
    // scores on the matrix cores: one accumulator per group of d/2 channels
    tile_f4 acc[2];
    acc[0] = tile_f4{0.0f, 0.0f, 0.0f, 0.0f};
    acc[1] = acc[0];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int gi = c / CPG, part = c % CPG;
      tile_h8 bop;
      if constexpr (F16T) {
        tile_u4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = R.k[gi][4 * part + i];
        bop = __builtin_bit_cast(tile_h8, u);
      } else {
        bop = tile_codes<QB>(R.k[gi], part, kmagic);
      }
      acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[c], bop, acc[gi], 0, 0, 0);
      acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_lo[c], bop, acc[gi], 0, 0, 0);
    }
    const int tok = grp * kTileG + ai;
    bool valid = hl < RT && tok < nt;
    if constexpr (IMPT) valid = valid && tok != frel;
    // the token's coefficients: scale / step on the product, zero - scale /
    // step on sum(q-hat) (for 8-bit codes, scale and zero)
    float ka[2], kz[2];
    if constexpr (!F16T) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        ka[gi] = lo_h(R.ksz[gi]) * (1.0f / kCodeStep<QB>);
        kz[gi] = hi_h(R.ksz[gi]) - (QB == 8 ? 0.0f : ka[gi]);
      }
    }
    float xv;
    if constexpr (F16T) {
      xv = acc[0][0] + acc[1][0];
    } else {
      xv = ka[0] * acc[0][0] + ka[1] * acc[1][0];
      xv += kz[0] * qs[0] + kz[1] * qs[1];
    }
    const float x = valid ? xv : -INFINITY;
    if constexpr (IMPT) {
      if (valid) p.sc16[scb + static_cast<int64_t>(hl) * p.cap16 + tok] = xv;
    }
    // lazy running maximum: moves only when a score exceeds it by more than
    // the headroom (also on the first scores of the wave)
    if (__builtin_amdgcn_ballot_w64(x > M + kTileHeadroom) != 0) {
      // the row maximum of each lane group is its head's (-inf on groups >= RT)
      const float mn = fmaxf(M, group_max<16>(x));
      const float f = mn > M ? fast_exp2(M - mn) : 1.0f;  // 0 when M was -inf
      l *= f;
      zz[0] *= f;
      zz[1] *= f;
      M = mn;
#pragma unroll
      for (int h = 0; h < RT; ++h) {
        const float fh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), 16 * h));
#pragma unroll
        for (int e = 0; e < 8; ++e) a[h][e] *= fh;
      }
    }
    // the probability and the weights of the value sums
    const float pr = fast_exp2(x - fmaxf(M, -FLT_MAX));
    l += pr;
    float w[2];
    if constexpr (F16T) {
      w[0] = pr;
      w[1] = pr;
    } else {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const float s = lo_h(R.vsz[gi]), z = hi_h(R.vsz[gi]);
        w[gi] = pr * s;
        zz[gi] += pr * z;
      }
    }
    if (hl < RT) {
      wbuf[wave][ai][0][hl] = w[0];
      wbuf[wave][ai][1][hl] = w[1];
    }
    __builtin_amdgcn_wave_barrier();
    // value sums: 8 channels per lane, VTPL tokens taken in pairs
    static_assert(VTPL % 2 == 0, "2-bit values pair the lane's tokens");
    // channel e += w * (the low or high half of word m)
    auto acc2 = [&](int e, const float (&w)[RT], uint32_t m, bool hi) {
      const float v = hi ? hi_h(m) : lo_h(m);
#pragma unroll
      for (int h = 0; h < RT; ++h) a[h][e] += w[h] * v;
    };
#pragma unroll
    for (int k = 0; k < VTPL; k += 2) {
      float wv[2][RT];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < RT; ++h) wv[j][h] = wbuf[wave][vs + (k + j) * VSLOTS][vg][h];
      if constexpr (QB == 2) {
        // tokens k and k + 1 in the low and high halves: each AND gives one
        // channel of both tokens
        const uint32_t x = R.v[k][0] | (R.v[k + 1][0] << 16), t = x >> 10;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t m = e < 5 ? (x & (0x00030003u << (2 * e))) : (t & (0x00030003u << (2 * (e - 5))));
          acc2(e, wv[0], m, false);
          acc2(e, wv[1], m, true);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t* vw = R.v[k + j];
          if constexpr (F16T) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc2(2 * i, wv[j], vw[i], false);
              acc2(2 * i + 1, wv[j], vw[i], true);
            }
          } else if constexpr (QB == 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {  // channels 2i, 2i + 1
              const uint32_t pr2 = __builtin_amdgcn_perm(magic, vw[i / 2], (i % 2) ? 0x04030402u : 0x04010400u);
              acc2(2 * i, wv[j], pr2, false);
              acc2(2 * i + 1, wv[j], pr2, true);
            }
          } else {
            // halves (c, c + 4): channels 0/4 and 1/5 in place, 2/6 and 3/7 after >> 8
            const uint32_t x = vw[0], t = x >> 8;
            const uint32_t m0 = x & 0x000F000Fu, m1 = x & 0x00F000F0u;
            const uint32_t m2 = t & 0x000F000Fu, m3 = t & 0x00F000F0u;
            acc2(0, wv[j], m0, false); acc2(4, wv[j], m0, true);
            acc2(1, wv[j], m1, false); acc2(5, wv[j], m1, true);
            acc2(2, wv[j], m2, false); acc2(6, wv[j], m2, true);
            acc2(3, wv[j], m3, false); acc2(7, wv[j], m3, true);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  for (int grp = wave; grp * kTileG < nt || grp == wave;) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      load(grp + 4 * (NS - 1), R[(i + NS - 1) % NS]);
      step(R[i], grp);
      grp += 4;
      if (grp * kTileG >= nt) break;
    }
  }

  // ---- wave partials: l and the zero-point sums over each head's 16 score
  // lanes (every lane of the group ends with its head's totals), value
  // slices over slots
  l = group_sum<16>(l);
  zz[0] = group_sum<16>(zz[0]);
  zz[1] = group_sum<16>(zz[1]);
  float zh[RT][2];
#pragma unroll
  for (int h = 0; h < RT; ++h) {
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
      zh[h][gi] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, zz[gi]), 16 * h));
#pragma unroll
    for (int e = 0; e < 8; ++e) a[h][e] = slot_sum<LPTV>(a[h][e]);
  }
  if (lane < LPTV) {
#pragma unroll
    for (int h = 0; h < RT; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        red[(wave * RT + h) * D + 8 * lane + e] = F16T ? a[h][e] : a[h][e] * tile_val_unit<QB>(e) + zh[h][vg];
  }
  if (lane % 16 == 0 && hl < RT) {
    sm[wave][hl] = M;
    red[4 * RT * D + wave * RT + hl] = l;
  }
  __syncthreads();
  // ---- block partial: the four waves rebased to their common maximum
  for (int i = tid; i < RT * D; i += kThreads) {
    const int h = i / D, c = i % D;
    const float mx = fmaxf(fmaxf(sm[0][h], sm[1][h]), fmaxf(sm[2][h], sm[3][h]));
    float o = 0.0f;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const float f = (sm[w4][h] == -INFINITY) ? 0.0f : fast_exp2(sm[w4][h] - mx);
      o += f * red[(w4 * RT + h) * D + c];
    }
    po[i] = o;
  }
  if (tid < RT) {
    const int h = tid;
    const float mx = fmaxf(fmaxf(sm[0][h], sm[1][h]), fmaxf(sm[2][h], sm[3][h]));
    float L = 0.0f;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4)
      L += (sm[w4][h] == -INFINITY) ? 0.0f : fast_exp2(sm[w4][h] - mx) * red[4 * RT * D + w4 * RT + h];
    pml[h] = make_float2(mx, L);
  }
}


#include "decode_tile_mv.hpp"

// Value sums on the matrix cores (tile_split_mv) for 2-bit retained codes of
// 2-4 heads: measured faster there (32K GQA layer, 4 heads: split kernel
// 22.4 -> 19.8-20.3 us). With 4-bit codes the path measured slower on the GQA
// batch (57.7-58.4 us at 168-170 registers against 53.5 us here: per-wave
// stamps show each 64-token step waiting on its MFMA chains and LDS round
// trips at two or three waves per SIMD); with one head 15 of the 16 MFMA rows
// idle and the importance-tier layer went 31.9 -> 35.0 us. Those keep
// tile_split.
__host__ __device__ constexpr bool tile_mv_of(int d, int bits, int rt) { return d == 128 && bits == 2 && rt >= 2; }
template <int D, int BITS, int RT>
constexpr bool tile_mv() { return tile_mv_of(D, BITS, RT); }
// These kernels run two blocks per compute unit (two waves per SIMD), although
// three fit their 166 registers: on the 32K GQA layer the split kernel took
// 17.4-17.5 us with two against 19.6-19.8 us with three (and 20.7 us with
// one); fewer waves per SIMD start their loops sooner and take a larger share
// of issue each.
constexpr int kMvBlocksPerCU = 2;

template <int D, int BITS, int IB, int RT>
__global__ __launch_bounds__(kThreads, (tile_mv<D, BITS, RT>() ? 2 : 3)) void decode_tile_kernel(const DecodeK p) {
  // block order as decode_split_kernel (split-major)
  const int S = p.S16 + p.Sq + p.Sb;
  const int ut = p.units * p.tiles;
  const int sd = blockIdx.x / ut;
  const int split = p.f16_first ? sd : ((sd < p.Sq) ? p.S16 + sd : sd - p.Sq);
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
  __shared__ float wbuf[4][kTileG][2][RT];
  constexpr bool kMv = tile_mv<D, BITS, RT>();  // value sums on the matrix cores
  __shared__ __attribute__((aligned(16))) unsigned char mvbuf[kMv ? 4 * MvStage<(BITS == 2 ? 2 : 4)>::BYTES : 16];

  if (split < p.S16) {
    tile_split<D, IB, RT, true>(p, unit, n, g, tile, split, bvec, red, sm_max, po, pml, wbuf);
  } else if constexpr (kMv) {
    tile_split_mv<BITS, RT>(p, unit, n, g, tile, split, bvec, red, sm_max, po, pml, mvbuf);
  } else {
    tile_split<D, BITS, RT, false>(p, unit, n, g, tile, split, bvec, red, sm_max, po, pml, wbuf);
  }
}
