// Head tiles of the low-bit tier with the value sums on the matrix cores
// (head dim 128, codes of 2 or 4 bits).
//
// velog notes "No Token Left Behind ...", section 3.4: with g query heads per
// kv head, decode attention over the retained codes is two small products per
// token block, scores = q-hat x keys and o = weights x values. tile_split runs
// the first on the matrix cores and the second on the vector ALUs (4 heads x 8
// channels of multiply-adds per token and lane). Here both run as
// v_mfma_f32_16x16x32_f16.
//
// A wave takes 64 tokens at a time: four 16-token groups of its share.
//  - Key scores as in tile_split, but with the tile's heads in A rows
//    0..RT-1 (A = q-hat hi and lo rows, B = the codes of 16 tokens); the four
//    groups' score tiles, held by lanes 0..15, are then moved
//    so that lane t holds token t's scores of every head (v_permlane16_swap,
//    v_permlane32_swap), and the softmax bookkeeping runs once per (token,
//    head) with every lane busy.
//  - Value product O[h][c] = sum_t W[h][t] * code[t][c] with W = p * value
//    scale: k = tokens, B = codes (column = channel), A = W as fp16 hi and lo
//    rows (about 22 bits of W). The codes enter as 1 + code * step, like the
//    keys' (tile_codes), and a second product against B = 1 sums W as the
//    matrix cores see it, so sum_t W * code = (O - that sum) / step holds
//    with no assumption on how they treat small W. A lane of B holds one channel across 8 tokens,
//    which the token-major cache does not give by loads. Each lane writes its
//    token's code row into LDS and a transposing read returns the channel
//    view: ds_read_b64_tr_b4 (lane j of a 16-lane group gets nibble j of the 16
//    rows its group points at) for 4-bit codes, ds_read_b64_tr_b8 (lane 8h + j
//    gets byte j of the rows of lanes h, h + 2, ..) for 2-bit codes. The
//    weights go through LDS as 4 heads x fp16 per token and come back in A-row
//    layout by ds_read_b64_tr_b16.
//  - W has to fit fp16 for any value scale: the running maximum M tracks
//    y = score + log2(max(value scales of the token, 2^-20)), so that
//    W = exp2(score - M) * scale <= exp2(y - M) <= 2^kMvHeadroom. Every sum is
//    taken against that M; any common reference gives the same softmax, and
//    exp2(score - M) <= 2^(kMvHeadroom + 20) stays finite in fp32.
// The zero-point part sum(p * zero) and the normaliser are kept per lane and
// head and summed over the wave at the end.
#pragma once

constexpr float kMvHeadroom = 15.0f;  // W <= 2^15 < fp16 max
constexpr float kMvScaleFloor = -20.0f;  // log2 of the smallest value scale M accounts for

template <int QB>
struct MvStage {
  static constexpr int ROWB = 128 * QB / 8;        // code bytes per token row (64 or 32)
  // row pitch in LDS: the 16 rows a transposing read gathers fall on distinct
  // bank pairs (72 B: 18 banks apart; 48 B: 12 banks apart, 16-byte rows)
  static constexpr int PITCH = QB == 4 ? 72 : 48;
  static constexpr int VBYTES = 64 * PITCH;        // staged rows of one wave
  static constexpr int WBYTES = 2 * 2 * 64 * 8;    // W: [group][hi/lo][token][4 heads] fp16
  static constexpr int BYTES = VBYTES + WBYTES;
};

// k-slot e (0..7) of a B operand <- token 8H + kMvPerm(e) of its 16-token
// group: the order the code conversion produces (4-bit: even nibbles, then odd)
template <int QB>
__device__ __forceinline__ constexpr int mv_perm(int e) {
  return QB == 4 ? ((e < 4) ? 2 * e : 2 * (e - 4) + 1) : e;
}

typedef int mv_v2i __attribute__((ext_vector_type(2)));
typedef short mv_v4s __attribute__((ext_vector_type(4)));
typedef unsigned int mv_u2 __attribute__((ext_vector_type(2)));
#define MV_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// 8 codes (one per token) in 8 bytes' crumb c (2-bit) or in a word's nibbles
// (4-bit) -> B operand, 1 + code * kCodeStep<QB> in k-slot order; magic =
// kCodeMagic<QB> (the encoding of tile_codes).
template <int QB>
__device__ __forceinline__ tile_h8 mv_codes(uint32_t w0, uint32_t w1, int c, uint32_t magic) {
  tile_u4 u;
  if constexpr (QB == 4) {  // w0: 8 nibbles = tokens 0..7, each moved to the top of its byte
    constexpr uint32_t kLo = 0x04010400u, kHi = 0x04030402u;
    const uint32_t lo = (w0 << 4) & 0xF0F0F0F0u, hi = w0 & 0xF0F0F0F0u;
    u[0] = __builtin_amdgcn_perm(magic, lo, kLo);
    u[1] = __builtin_amdgcn_perm(magic, lo, kHi);
    u[2] = __builtin_amdgcn_perm(magic, hi, kLo);
    u[3] = __builtin_amdgcn_perm(magic, hi, kHi);
  } else {  // bytes of w0, w1 = tokens 0..7; crumb c of each as 0x3C | code over a zero byte
    constexpr uint32_t kB01 = 0x01040004u, kB23 = 0x03040204u;
    const uint32_t y0 = ((w0 >> (2 * c)) & 0x03030303u) | magic;
    const uint32_t y1 = ((w1 >> (2 * c)) & 0x03030303u) | magic;
    u[0] = __builtin_amdgcn_perm(0u, y0, kB01);
    u[1] = __builtin_amdgcn_perm(0u, y0, kB23);
    u[2] = __builtin_amdgcn_perm(0u, y1, kB01);
    u[3] = __builtin_amdgcn_perm(0u, y1, kB23);
  }
  (void)w1;
  (void)c;
  return __builtin_bit_cast(tile_h8, u);
}

// Channel of column n of value tile vt (8 tiles of 16 channels).
template <int QB>
__device__ __forceinline__ constexpr int mv_chan(int vt, int n) {
  // 4-bit: tile vt = channels 16 vt + n; 2-bit: tile (kappa = vt / 4, crumb
  // c = vt % 4), column n = 8 h + j -> channel 64 kappa + 32 h + 4 j + c
  return QB == 4 ? 16 * vt + n : 64 * (vt / 4) + 32 * (n / 8) + 4 * (n % 8) + (vt % 4);
}

template <int QB, int RT>
__device__ __forceinline__ void tile_split_mv(const DecodeK& p, int unit, int n, int g, int tile, int split,
                                              const float* bvec, float* red, float (*sm)[RT], float* po,
                                              float2* pml, unsigned char* mvbuf) {
  constexpr int D = 128, NCH = 4, CPG = 2, G = 64;
  using S_t = MvStage<QB>;
  constexpr int ROWB = S_t::ROWB, PITCH = S_t::PITCH;
  constexpr int KB = CPG * 8 * QB / 8, KW = (KB + 3) / 4;  // key bytes / words per lane and half-row group
  constexpr int VW = ROWB / 4;                            // value row words per lane
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int ai = lane % 16, ar = lane / 16;  // MFMA row / k block of this lane
  unsigned char* vst = mvbuf + wave * S_t::BYTES;
  unsigned char* wst = vst + S_t::VBYTES;

  // ---- block range and buffer resources (retained tier)
  const int t0 = (split - p.S16) * p.Cq;
  const int t1 = min(p.nq, t0 + p.Cq);
  const int nt = max(t1 - t0, 0);
  const int64_t ub = static_cast<int64_t>(unit) * p.capq + t0;
  const Rsrc rk = make_rsrc(p.kq + ub * ROWB, static_cast<uint32_t>(nt) * ROWB);
  const Rsrc rv = make_rsrc(p.vq + ub * ROWB, static_cast<uint32_t>(nt) * ROWB);
  const Rsrc rks = make_rsrc(p.ksz + ub * 2, static_cast<uint32_t>(nt) * 8);
  const Rsrc rvs = make_rsrc(p.vsz + ub * 2, static_cast<uint32_t>(nt) * 8);
  const int ngrp = (nt + kTileG - 1) / kTileG;
  const int mygrp = ngrp > wave ? (ngrp - wave + 3) / 4 : 0;  // groups wave, wave + 4, ...
  const int nss = (mygrp + 3) / 4;                              // supersteps of 4 groups

  // token of lane t = 16 r + i in superstep s: group wave + 4 (4 s + r), row i
  auto lane_tok = [&](int s) -> uint32_t {
    return static_cast<uint32_t>((wave + 4 * (4 * s + lane / 16)) * kTileG + lane % 16);
  };

  // ---- q and b first (as tile_split)
  const float qscale = kLog2e / sqrtf(static_cast<float>(D));
  float qv[NCH][8], bv[NCH][8];
  tile_load_qb<D, RT>(p, n, g, tile, bvec, ai, ar, qv, bv);

  // ---- register sets, each refilled for the next superstep as soon as it
  // has been consumed (so its loads have a whole superstep to arrive)
  uint32_t kr[4][2][KW];  // keys of the 4 groups (tile_split layout)
  uint32_t vr[VW];        // this lane's token row of value codes
  uint32_t ksz[2], vsz[2];
  auto load_key_group = [&](int s, int r) {
    const uint32_t tk = static_cast<uint32_t>((wave + 4 * (4 * s + r)) * kTileG + ai);
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) tile_load<KB>(rk, tk * ROWB + (gi * G + 8 * CPG * ar) * QB / 8, kr[r][gi]);
  };
  auto load_keys = [&](int s) {
#pragma unroll
    for (int r = 0; r < 4; ++r) load_key_group(s, r);
  };
  auto load_vals = [&](int s) {
    const uint32_t tv = lane_tok(s);
#pragma unroll
    for (int i = 0; i < VW / 4; ++i) {
      const Words<4> w = bload<4>(rv, tv * ROWB + 16 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) vr[4 * i + e] = w.w[e];
    }
  };
  auto load_sz = [&](int s) {
    const uint32_t tv = lane_tok(s);
    const Words<2> a = bload<2>(rks, tv * 8), b = bload<2>(rvs, tv * 8);
    ksz[0] = a.w[0]; ksz[1] = a.w[1];
    vsz[0] = b.w[0]; vsz[1] = b.w[1];
  };
  load_vals(0);
  load_keys(0);

  // ---- q-hat as MFMA A operands, per-group sums of q-hat (as tile_split)
  tile_h8 qa_hi[NCH], qa_lo[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int base = tile_chan<D, 16>(c, ar, 0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ch = tile_chan<D, QB>(c, ar, e);
      const float qe = qv[c][ch - base] * __builtin_amdgcn_rcpf(bv[c][ch - base]) * qscale;
      const float q = ai < RT ? qe : 0.0f;
      const _Float16 hi = static_cast<_Float16>(q);
      qa_hi[c][e] = hi;
      qa_lo[c][e] = static_cast<_Float16>(q - static_cast<float>(hi));
    }
  }
  float qs[RT][2];
  tile_qsums<NCH, RT>(qa_hi, qa_lo, qs);

  // ---- state: per head the reference M (uniform); per lane the normaliser
  // and zero-point sums; value tiles (lanes 0..15 = heads 0..3 x 16 channels)
  float M[RT], l[RT], zz[RT][2];
  tile_f4 Dv[8], Dw[2];  // value tiles; W summed against B = 1 per channel group
#pragma unroll
  for (int h = 0; h < RT; ++h) {
    M[h] = -INFINITY;
    l[h] = 0.0f;
    zz[h][0] = zz[h][1] = 0.0f;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) Dv[t] = tile_f4{0.0f, 0.0f, 0.0f, 0.0f};
  Dw[0] = Dv[0];
  Dw[1] = Dv[0];
  const tile_h8 ones = static_cast<tile_h8>(static_cast<_Float16>(1.0f));

  const uint32_t kmagic = opaque(kCodeMagic<QB>);
  const int kb = lane / 16, li = lane % 16;
  // this lane as a source of the W reads: row of its group for read r, half H
  // (one lane base; every (group, hi/lo, H, r) is a constant offset from it,
  // which the reads carry in their offset field: perm(4 r + i) - perm(i) is
  // 4 r for 2-bit codes and r for 4-bit codes)
  unsigned char* const wbase = wst + (16 * kb + mv_perm<QB>(li / 4)) * 8;
  auto w_src = [&](int gi, int hl, int H, int r) -> unsigned char* {
    return wbase + ((gi * 2 + hl) * 64 + 8 * H + (QB == 4 ? r : 4 * r)) * 8;
  };
  // this lane as a source of the 2-bit code reads: row 16 kb + 8 H + i of
  // chunk 2 kp + h (lane = 16 kb + 2 i + h), again a base plus constants
  const unsigned char* const cbase = vst + (16 * kb + li / 2) * PITCH + 8 * (li % 2);

  for (int s = 0; s < nss; ++s) {
    // this superstep's scales, loaded here rather than one superstep ahead: a
    // prefetched copy is a loaded value carried around the loop, and the
    // compiler moved it between registers at the loop edge behind a wait for
    // every load in flight; issued first, their own wait at the softmax does
    // not cover the prefetches issued after them. (Issuing the next
    // superstep's scales right after this one's last use, into the same
    // registers, avoids the copy but measured no faster: 32K GQA layer
    // 17.5-17.6 against 17.4-17.5 us.)
    load_sz(s);
    // (1) value code rows into LDS (row = lane), then the next superstep's
    // rows into the same registers
    if constexpr (QB == 4) {
#pragma unroll
      for (int i = 0; i < VW / 2; ++i)
        *reinterpret_cast<uint2*>(vst + lane * PITCH + 8 * i) = make_uint2(vr[2 * i], vr[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < VW / 4; ++i)
        *reinterpret_cast<uint4*>(vst + lane * PITCH + 16 * i) =
            make_uint4(vr[4 * i], vr[4 * i + 1], vr[4 * i + 2], vr[4 * i + 3]);
    }
    load_vals(s + 1);  // unconditional: past the range the loads return zeros, and exact wait counts need them

    // (2) key scores of the 4 groups on the matrix cores, two groups at a time,
    // each group's key registers refilled for the next superstep once used;
    // (3) lane t = 16 r + i takes token i of group r: row 0 (lanes 0..15) of
    // groups 2 q and 2 q + 1 paired by v_permlane16_swap, the pairs by
    // v_permlane32_swap
    auto group_scores = [&](int r, tile_f4 (&a)[2]) {
      a[0] = tile_f4{0.0f, 0.0f, 0.0f, 0.0f};
      a[1] = a[0];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int gi = c / CPG, part = c % CPG;
        const tile_h8 bop = tile_codes<QB>(kr[r][gi], part, kmagic);
        a[gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[c], bop, a[gi], 0, 0, 0);
        a[gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_lo[c], bop, a[gi], 0, 0, 0);
      }
      load_key_group(s + 1, r);
    };
    uint32_t pair[2][2][RT];  // [group pair][channel group][head]
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      tile_f4 a0[2], a1[2];
      group_scores(2 * q2, a0);
      group_scores(2 * q2 + 1, a1);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int h = 0; h < RT; ++h) {
          const auto t = __builtin_amdgcn_permlane16_swap(f2u(a0[gi][h]), f2u(a1[gi][h]), false, false);
          pair[q2][gi][h] = static_cast<uint32_t>(t[0]);
        }
    }
    float x[2][RT];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int h = 0; h < RT; ++h) {
        const auto t = __builtin_amdgcn_permlane32_swap(pair[0][gi][h], pair[1][gi][h], false, false);
        x[gi][h] = u2f(static_cast<uint32_t>(t[0]));
      }

    // (4) scores, the lazy reference, probabilities and weights
    const int tok = static_cast<int>(lane_tok(s));
    const bool valid = tok < nt;
    // key coefficients as in tile_split: scale / step, zero - scale / step
    const float ka0 = lo_h(ksz[0]) * (1.0f / kCodeStep<QB>), ka1 = lo_h(ksz[1]) * (1.0f / kCodeStep<QB>);
    const float kz0 = hi_h(ksz[0]) - ka0, kz1 = hi_h(ksz[1]) - ka1;
    const float sv0 = lo_h(vsz[0]), sv1 = lo_h(vsz[1]), zv0 = hi_h(vsz[0]), zv1 = hi_h(vsz[1]);
    const float yoff = fmaxf(__builtin_amdgcn_logf(fmaxf(sv0, sv1)), kMvScaleFloor);
    float xs[RT], y[RT];
    bool need = false;
#pragma unroll
    for (int h = 0; h < RT; ++h) {
      const float xv = ka0 * x[0][h] + ka1 * x[1][h] + kz0 * qs[h][0] + kz1 * qs[h][1];
      xs[h] = valid ? xv : -INFINITY;
      y[h] = xs[h] + yoff;
      need |= y[h] > M[h] + kMvHeadroom;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int h = 0; h < RT; ++h) {
        const float mn = fmaxf(M[h], wave_max(y[h]));
        if (mn > M[h]) {
          const float f = fast_exp2(M[h] - mn);  // 0 when M was -inf
          l[h] *= f;
          zz[h][0] *= f;
          zz[h][1] *= f;
#pragma unroll
          for (int t = 0; t < 8; ++t) Dv[t][h] *= f;
          Dw[0][h] *= f;
          Dw[1][h] *= f;
          M[h] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mn)));  // uniform
        }
      }
    }
    uint32_t wh[2][2][2];  // [group][hi/lo][word of 4 heads]
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl) wh[gi][hl][0] = wh[gi][hl][1] = 0u;
#pragma unroll
    for (int h = 0; h < RT; ++h) {
      const float pr = fast_exp2(xs[h] - fmaxf(M[h], -FLT_MAX));
      l[h] += pr;
      zz[h][0] += pr * zv0;
      zz[h][1] += pr * zv1;
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const float w = pr * (gi ? sv1 : sv0);
        const _Float16 whi = static_cast<_Float16>(w);
        const _Float16 wlo = static_cast<_Float16>(w - static_cast<float>(whi));
        wh[gi][0][h / 2] |= static_cast<uint32_t>(__builtin_bit_cast(uint16_t, whi)) << (16 * (h % 2));
        wh[gi][1][h / 2] |= static_cast<uint32_t>(__builtin_bit_cast(uint16_t, wlo)) << (16 * (h % 2));
      }
    }
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
        *reinterpret_cast<uint2*>(wst + ((gi * 2 + hl) * 64 + lane) * 8) = make_uint2(wh[gi][hl][0], wh[gi][hl][1]);
    __builtin_amdgcn_wave_barrier();

    // (5) W back in A-row layout (row m = head, k-slot e = token 8H + perm(e)),
    // each (group, H) pair read right before its MFMAs; the results are taken
    // as whole 32-bit words: unpacking them element by element into an fp16
    // vector compiled into element 0 repeated
    auto read_w = [&](int gi, int H, tile_h8& whi, tile_h8& wlo) {
      const mv_u2 a = __builtin_bit_cast(mv_u2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(MV_LDS(mv_v4s, w_src(gi, 0, H, 0))));
      const mv_u2 b = __builtin_bit_cast(mv_u2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(MV_LDS(mv_v4s, w_src(gi, 0, H, 1))));
      const mv_u2 c = __builtin_bit_cast(mv_u2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(MV_LDS(mv_v4s, w_src(gi, 1, H, 0))));
      const mv_u2 d = __builtin_bit_cast(mv_u2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(MV_LDS(mv_v4s, w_src(gi, 1, H, 1))));
      whi = __builtin_bit_cast(tile_h8, tile_u4{a[0], a[1], b[0], b[1]});
      wlo = __builtin_bit_cast(tile_h8, tile_u4{c[0], c[1], d[0], d[1]});
    };

    // (6) value tiles: codes transposed out of LDS, W x codes on the matrix cores
    if constexpr (QB == 4) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        mv_v2i cw[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          cw[v] = __builtin_amdgcn_ds_read_tr4_b64_v2i32(MV_LDS(mv_v2i, vst + lane * PITCH + 8 * (4 * gi + v)));
#pragma unroll
        for (int H = 0; H < 2; ++H) {
          tile_h8 whi, wlo;
          read_w(gi, H, whi, wlo);
          Dw[gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(whi, ones, Dw[gi], 0, 0, 0);
          Dw[gi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wlo, ones, Dw[gi], 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int vt = 4 * gi + v;
            const tile_h8 bop = mv_codes<4>(static_cast<uint32_t>(cw[v][H]), 0u, 0, kmagic);
            Dv[vt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(whi, bop, Dv[vt], 0, 0, 0);
            Dv[vt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wlo, bop, Dv[vt], 0, 0, 0);
          }
        }
      }
    } else {
#pragma unroll
      for (int H = 0; H < 2; ++H)
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const unsigned char* src = cbase + 8 * H * PITCH + 16 * kp;
          const mv_v2i cw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(MV_LDS(mv_v2i, src));
          tile_h8 whi, wlo;
          read_w(kp, H, whi, wlo);
          Dw[kp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(whi, ones, Dw[kp], 0, 0, 0);
          Dw[kp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wlo, ones, Dw[kp], 0, 0, 0);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const tile_h8 bop = mv_codes<2>(static_cast<uint32_t>(cw[0]), static_cast<uint32_t>(cw[1]), c, kmagic);
            const int vt = 4 * kp + c;
            Dv[vt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(whi, bop, Dv[vt], 0, 0, 0);
            Dv[vt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wlo, bop, Dv[vt], 0, 0, 0);
          }
        }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- wave partials: normaliser and zero-point sums over all lanes; value
  // tiles and W sums are already summed over the wave's tokens (lanes 0..15;
  // every column of Dw holds the same sum), sum_t W * code = (Dv - Dw) / step
#pragma unroll
  for (int h = 0; h < RT; ++h) {
    l[h] = wave_sum(l[h]);
    zz[h][0] = wave_sum(zz[h][0]);
    zz[h][1] = wave_sum(zz[h][1]);
  }
  if (lane < 16) {
#pragma unroll
    for (int vt = 0; vt < 8; ++vt) {
      const int ch = mv_chan<QB>(vt, lane);
#pragma unroll
      for (int h = 0; h < RT; ++h)
        red[(wave * RT + h) * D + ch] = (Dv[vt][h] - Dw[ch / G][h]) * (1.0f / kCodeStep<QB>) + zz[h][ch / G];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < RT; ++h) {
      sm[wave][h] = M[h];
      red[4 * RT * D + wave * RT + h] = l[h];
    }
  }
  __syncthreads();
  // ---- block partial: the four waves rebased to their common reference
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
