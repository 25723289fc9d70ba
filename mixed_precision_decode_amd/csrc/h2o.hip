// Heavy-hitter bookkeeping, important-set re-selection and demotion.
//
// velog notes "No Token Left Behind ...", one-line summary and Key
// contributions 1): the importance-based eviction (H2O) decides which tokens
// stay at high precision; the tokens it would evict are kept as low-bit
// codes instead. paperlayer summary of arXiv 2402.18096, section 5:
// heavy hitters (largest accumulated attention) plus local (recent) tokens.
// Ranking key: accumulated attention descending, token position ascending.
//
// Decode: one block per (sequence, kv head) adds this step's probabilities,
// finds the one candidate that falls out of the top-`heavy` (an argmin over
// heavy+1 candidates) and quantizes its key and value rows into the next
// low-bit slot.
// Prefill: a radix select over 32-bit order-preserving keys finds the
// top-`heavy` threshold of [0, T-recent), ties are taken by ascending
// position, and block-wide prefix sums assign ascending-position slots in
// both tiers; a second, token-parallel kernel moves the rows (fp16 copy or
// quantization) - the HBM-bound part.
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"
#include "h2o_common.hpp"

#include <climits>

namespace mikv {

// ------------------------------------------------------------------ decode
// All slot loads of the block are issued at once (up to kH2OSlots per
// thread, the common case), so the select costs one memory round trip and the
// demotion a second one.
constexpr int kH2OSlots = 16;
// The cache views of the H2O args as the shared select/demote code takes them.
static __device__ __forceinline__ H2OView h2o_view(const H2OArgs& a, int IB) {
  H2OView v;
  v.cap16 = a.cap16; v.capq = a.capq; v.len = a.len; v.recent = a.recent; v.imp_bits = IB;
  v.k16 = a.k16; v.v16 = a.v16; v.pos16 = a.pos16; v.acc16 = a.acc16; v.free16 = a.free16;
  v.kimp = a.kimp; v.vimp = a.vimp;
  v.kimpsz = reinterpret_cast<uint32_t*>(a.kimpsz);
  v.vimpsz = reinterpret_cast<uint32_t*>(a.vimpsz);
  v.kq = a.kq; v.vq = a.vq;
  v.ksz = reinterpret_cast<uint32_t*>(a.ksz);
  v.vsz = reinterpret_cast<uint32_t*>(a.vsz);
  v.posq = a.posq; v.demoted_pos = a.demoted_pos;
  v.key_tile = a.key_tile;
  v.kcsz = reinterpret_cast<uint32_t*>(a.kcsz);
  v.kbuf = a.kbuf; v.vbuf = a.vbuf; v.posbuf = a.posbuf;
  return v;
}

template <int D, int BITS, int NL, int IB, bool KT>
__global__ __launch_bounds__(256) void h2o_decode_kernel(H2OArgs a) {
  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base16 = static_cast<int64_t>(unit) * a.cap16;
  const float* accin = a.acc16 + base16;  // rewritten below, so not restrict
  const float* __restrict__ p16 = a.p16 + base16;
  const int32_t* __restrict__ pos16 = a.pos16 + base16;
  const int fr = a.free16[unit];
  const int limit = a.len - a.recent;  // candidates: pos < limit
  Worst w;
  auto consider = [&](int s, float prev, float pp, int pos) {
    if (s == fr) { prev = 0.0f; pos = a.len - 1; }
    const float v = prev + pp;
    a.acc16[base16 + s] = v;
    if (pos < limit) w.consider(v, pos, s);
  };
  if (a.cap16 <= kH2OSlots * 256) {
    float av[kH2OSlots], pv[kH2OSlots];
    int qv[kH2OSlots];
#pragma unroll
    for (int k = 0; k < kH2OSlots; ++k) {
      const int s = tid + k * 256;
      if (s < a.cap16) { av[k] = accin[s]; pv[k] = p16[s]; qv[k] = pos16[s]; }
    }
#pragma unroll
    for (int k = 0; k < kH2OSlots; ++k) {
      const int s = tid + k * 256;
      if (s < a.cap16) consider(s, av[k], pv[k], qv[k]);
    }
  } else {
    for (int s = tid; s < a.cap16; s += 256) consider(s, accin[s], p16[s], pos16[s]);
  }
  h2o_select_demote<D, BITS, NL, KT>(w, h2o_view(a, IB), unit);
}

// ------------------------------------------------------------------ prefill
// One block of kSelThreads per (sequence, kv head). After the radix select,
// positions are visited in chunks of kSelThreads * kSelRun; each thread takes
// kSelRun consecutive positions, so a chunk costs two block scans (ties, then
// the kept positions).
constexpr int kSelThreads = 1024;
constexpr int kSelRun = 8;

__global__ __launch_bounds__(kSelThreads) void h2o_prefill_select_kernel(H2OArgs a, int T, int32_t* map) {
  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  const float* acc0 = a.src_acc0 + static_cast<int64_t>(unit) * T;
  const int ncand = T - a.recent;
  const int H = a.heavy;
  // threshold key of the H-th best candidate; `need` of its ties are kept
  uint32_t tau = 0xFFFFFFFFu;
  int need = 0;
  if (H > 0) {
    block_radix_topm<kSelThreads, 32>(ncand, H, [&](int i, uint32_t* key) {
      *key = float_key(acc0[i]);
      return true;
    }, &tau, &need);
  }
  // ascending-position slot assignment in both tiers
  int eq_seen = 0, kept = 0;
  const int64_t base16 = static_cast<int64_t>(unit) * a.cap16;
  const int64_t baseq = static_cast<int64_t>(unit) * a.capq;
  int32_t* umap = map + static_cast<int64_t>(unit) * T;
  // per-channel key tiles: retained ranks from nq0 on start the buffer
  const int nq0 = a.key_tile ? (T - (a.cap16 - 1)) / kKeyTile * kKeyTile : INT_MAX;
  for (int p0 = 0; p0 < T; p0 += kSelThreads * kSelRun) {
    const int base = p0 + tid * kSelRun;
    float av[kSelRun];
    uint32_t key[kSelRun];
    int neq = 0;
#pragma unroll
    for (int j = 0; j < kSelRun; ++j) {
      const int p = base + j;
      av[j] = (p < T) ? acc0[p] : 0.0f;
      key[j] = float_key(av[j]);
      neq += (H > 0 && p < ncand && key[j] == tau) ? 1 : 0;
    }
    int eq_tot;
    int eq_rank = eq_seen + block_scan_add<kSelThreads>(neq, &eq_tot);
    eq_seen += eq_tot;
    bool keep[kSelRun];
    int nk = 0;
#pragma unroll
    for (int j = 0; j < kSelRun; ++j) {
      const int p = base + j;
      const bool cand = p < ncand;
      const bool eq = H > 0 && cand && key[j] == tau;
      keep[j] = p < T && (!cand || (H > 0 && (key[j] > tau || (eq && eq_rank < need))));
      eq_rank += eq ? 1 : 0;
      nk += keep[j] ? 1 : 0;
    }
    int k_tot;
    int krank = kept + block_scan_add<kSelThreads>(nk, &k_tot);
    // slots are bounds-checked so that a selection error can only show up
    // as a wrong result (map entry INT_MIN = not stored)
#pragma unroll
    for (int j = 0; j < kSelRun; ++j) {
      const int p = base + j;
      if (p < T) {
        if (keep[j]) {
          const int slot = krank++;
          const bool ok = slot < a.cap16 - 1;
          if (ok) {
            a.pos16[base16 + slot] = p;
            a.acc16[base16 + slot] = av[j];
          }
          umap[p] = ok ? slot : INT_MIN;
        } else {
          // positions before p that were not kept
          const int slot = p - krank;
          const bool ok = slot < a.capq;
          if (ok) {
            if (slot < nq0) a.posq[baseq + slot] = p;
            else a.posbuf[static_cast<int64_t>(unit) * kKeyTile + (slot - nq0)] = p;
          }
          umap[p] = ok ? -1 - slot : INT_MIN;
        }
      }
    }
    kept += k_tot;
  }
  if (tid == 0) {
    a.free16[unit] = a.cap16 - 1;
    a.pos16[base16 + a.cap16 - 1] = -1;
    a.acc16[base16 + a.cap16 - 1] = 0.0f;
  }
  // the free slot's rows start as zeros: decode reads them (masked), so they
  // must hold finite values
  if (a.imp_bits == 16) {
    for (int i = tid; i < a.d / 8; i += kSelThreads) {
      const int64_t o = (base16 + a.cap16 - 1) * a.d + 8 * i;
      *reinterpret_cast<uint4*>(a.k16 + o) = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(a.v16 + o) = make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
    // codes 0 with (scale, zero) = (0, 0): the free slot reads as zeros
    const int cbi = a.d * a.imp_bits / 8, ng = a.d / a.group;
    for (int i = tid; i < cbi / 4; i += kSelThreads) {
      const int64_t o = (base16 + a.cap16 - 1) * cbi + 4 * i;
      *reinterpret_cast<uint32_t*>(a.kimp + o) = 0u;
      *reinterpret_cast<uint32_t*>(a.vimp + o) = 0u;
    }
    for (int i = tid; i < ng; i += kSelThreads) {
      reinterpret_cast<uint32_t*>(a.kimpsz)[(base16 + a.cap16 - 1) * ng + i] = 0u;
      reinterpret_cast<uint32_t*>(a.vimpsz)[(base16 + a.cap16 - 1) * ng + i] = 0u;
    }
  }
}

#ifndef MIKV_SCATTER_BLOCKS
#define MIKV_SCATTER_BLOCKS 4096
#endif
// 16 blocks of 256 threads per compute unit (measured best among 1024-65536)
constexpr int64_t kScatterBlocks = MIKV_SCATTER_BLOCKS;

template <int D, int BITS, int NL, int IB, bool KT>
__global__ __launch_bounds__(256) void h2o_prefill_scatter_kernel(H2OArgs a, int T,
                                                                  const int32_t* map) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  constexpr int CB = D * BITS / 8;
  constexpr int GPT = D / (8 * NL);
  const int lane = threadIdx.x % LPR;
  const int64_t n_rows = static_cast<int64_t>(a.batch) * a.hkv * T;
  const int64_t step = static_cast<int64_t>(gridDim.x) * RPB;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR;
  if (r0 >= n_rows) return;
  const bool bal = a.src_b != nullptr;
  // a row is tracked as (row, unit, position); the grid stride advances all
  // three without a division per row
  const int64_t su = step / T;
  const int sr = static_cast<int>(step % T);
  auto advance = [&](int64_t& r, int64_t& u, int& t) {
    r += step;
    u += su;
    t += sr;
    if (t >= T) {
      t -= T;
      ++u;
    }
  };
  struct Row {
    uint4 k, v;
    float4 b0, b1;
    int s;
  };
  auto load = [&](int64_t r, int64_t u, Row& R) {
    R.k = *reinterpret_cast<const uint4*>(a.src_k + r * D + lane * 8);
    R.v = *reinterpret_cast<const uint4*>(a.src_v + r * D + lane * 8);
    R.s = map[r];
    if (bal) {
      const float4* bb = reinterpret_cast<const float4*>(a.src_b + u * D + lane * 8);
      R.b0 = bb[0];
      R.b1 = bb[1];
    }
  };
  auto process = [&](int64_t unit, const Row& R) {
    float kx[8], vx[8];
    kx[0] = lo_h(R.k.x); kx[1] = hi_h(R.k.x); kx[2] = lo_h(R.k.y); kx[3] = hi_h(R.k.y);
    kx[4] = lo_h(R.k.z); kx[5] = hi_h(R.k.z); kx[6] = lo_h(R.k.w); kx[7] = hi_h(R.k.w);
    vx[0] = lo_h(R.v.x); vx[1] = hi_h(R.v.x); vx[2] = lo_h(R.v.y); vx[3] = hi_h(R.v.y);
    vx[4] = lo_h(R.v.z); vx[5] = hi_h(R.v.z); vx[6] = lo_h(R.v.w); vx[7] = hi_h(R.v.w);
    uint32_t kw[4] = {R.k.x, R.k.y, R.k.z, R.k.w};
    if (bal) {
      const float bb[8] = {R.b0.x, R.b0.y, R.b0.z, R.b0.w, R.b1.x, R.b1.y, R.b1.z, R.b1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) kx[i] = h2f(f2h(mul_rn(kx[i], bb[i])));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kw[i] = static_cast<uint32_t>(f2h(kx[2 * i])) | (static_cast<uint32_t>(f2h(kx[2 * i + 1])) << 16);
    }
    // R.s is the same on every lane of a row and the group reductions of
    // quantize8 stay inside a row, so the branches keep rows whole
    if (R.s >= 0) {
      if constexpr (IB == 16) {
        const int64_t o16 = (unit * a.cap16 + R.s) * D + lane * 8;
        *reinterpret_cast<uint4*>(a.k16 + o16) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
        *reinterpret_cast<uint4*>(a.v16 + o16) = R.v;
      } else {
        // reduced-precision importance tier: the row is stored as IB-bit codes
        constexpr int CBI = D * IB / 8;
        uint32_t kszw, vszw, kc[8], vc[8], kw2[2], vw2[2];
        quantize8_codes<IB, NL>(kx, &kszw, kc);
        quantize8_codes<IB, NL>(vx, &vszw, vc);
        pack8<IB>(kc, kw2);
        pack8<IB>(vc, vw2);
        const int64_t si = unit * a.cap16 + R.s;
        store_codes8w<IB>(a.kimp + si * CBI, lane, kw2);
        store_codes8w<IB>(a.vimp + si * CBI, lane, vw2);
        if (lane % NL == 0) {
          reinterpret_cast<uint32_t*>(a.kimpsz)[si * GPT + lane / NL] = kszw;
          reinterpret_cast<uint32_t*>(a.vimpsz)[si * GPT + lane / NL] = vszw;
        }
      }
    } else if (KT && R.s != INT_MIN) {
      // per-channel key tiles: values per token into the tile slots (the
      // keys follow per tile in h2o_key_tile_kernel); the last (T - B) mod 64
      // retained pairs go to the buffer as fp16
      const int slot = -1 - R.s;
      const int nq0 = (T - (a.cap16 - 1)) / kKeyTile * kKeyTile;
      if (slot < nq0) {
        uint32_t vszw;
        const uint32_t vp = quantize8<BITS, NL>(vx, &vszw);
        const int64_t qs = unit * a.capq + slot;
        store_codes8<BITS>(a.vq + qs * CB, lane, vp);
        if (lane % NL == 0) reinterpret_cast<uint32_t*>(a.vsz)[qs * GPT + lane / NL] = vszw;
      } else {
        const int64_t ob = (unit * kKeyTile + (slot - nq0)) * D + lane * 8;
        *reinterpret_cast<uint4*>(a.kbuf + ob) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
        *reinterpret_cast<uint4*>(a.vbuf + ob) = R.v;
      }
    } else if (R.s != INT_MIN) {
      uint32_t kszw, vszw;
      const uint32_t kp = quantize8<BITS, NL>(kx, &kszw);
      const uint32_t vp = quantize8<BITS, NL>(vx, &vszw);
      const int64_t qs = unit * a.capq + (-1 - R.s);
      store_codes8<BITS>(a.kq + qs * CB, lane, kp);
      store_codes8<BITS>(a.vq + qs * CB, lane, vp);
      if (lane % NL == 0) {
        reinterpret_cast<uint32_t*>(a.ksz)[qs * GPT + lane / NL] = kszw;
        reinterpret_cast<uint32_t*>(a.vsz)[qs * GPT + lane / NL] = vszw;
      }
    }
  };
  // two register sets in turn: the loads of the next row are in flight
  // while the current one is processed; past the end a load repeats the
  // current row (a valid address) and its result is not used
  int64_t ra = r0, ua = r0 / T;
  int ta = static_cast<int>(r0 % T);
  Row A, B;
  load(ra, ua, A);
  for (;;) {
    int64_t rb = ra, ub = ua;
    int tb = ta;
    advance(rb, ub, tb);
    const bool hb = rb < n_rows;  // the same for every lane of a row
    load(hb ? rb : ra, hb ? ub : ua, B);
    process(ua, A);
    if (!hb) break;
    ra = rb;
    ua = ub;
    ta = tb;
    advance(ra, ua, ta);
    const bool ha = ra < n_rows;
    load(ha ? ra : rb, ha ? ua : ub, A);
    process(ub, B);
    if (!ha) break;
  }
}

// Prefill key tiles: one block per (sequence, kv head, tile of 64 retained
// positions). The balanced key rows of the tile's positions (posq, written by
// the select kernel) are gathered into LDS and quantized per channel.
template <int D, int BITS>
__global__ __launch_bounds__(256) void h2o_key_tile_kernel(H2OArgs a, int T, int tiles) {
  __shared__ uint16_t s_x[kKeyTile * D];
  __shared__ uint8_t s_c[kKeyTile * D];
  __shared__ int s_pos[kKeyTile];
  constexpr int LPR = D / 8, CB = D * BITS / 8;
  const int unit = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int tid = threadIdx.x;
  const int64_t q0 = static_cast<int64_t>(unit) * a.capq + static_cast<int64_t>(tile) * kKeyTile;
  // positions are clamped into the prompt, so that a selection error could
  // only give a wrong result, never a read outside src_k
  if (tid < kKeyTile) s_pos[tid] = min(max(a.posq[q0 + tid], 0), T - 1);
  __syncthreads();
  const float* bvec = a.src_b ? a.src_b + static_cast<int64_t>(unit) * D : nullptr;
  for (int i = tid; i < kKeyTile * LPR; i += 256) {
    const int t = i / LPR, lane = i % LPR;
    const int64_t r = static_cast<int64_t>(unit) * T + s_pos[t];
    uint4 w = *reinterpret_cast<const uint4*>(a.src_k + r * D + lane * 8);
    if (bvec) {
      uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = h2f(f2h(mul_rn(lo_h(ww[j]), bvec[lane * 8 + 2 * j])));
        const float hi = h2f(f2h(mul_rn(hi_h(ww[j]), bvec[lane * 8 + 2 * j + 1])));
        ww[j] = static_cast<uint32_t>(f2h(lo)) | (static_cast<uint32_t>(f2h(hi)) << 16);
      }
      w = make_uint4(ww[0], ww[1], ww[2], ww[3]);
    }
    *reinterpret_cast<uint4*>(s_x + t * D + lane * 8) = w;
  }
  __syncthreads();
  quantize_key_tile<D, BITS>(s_x, s_c, a.kq + q0 * CB,
                             reinterpret_cast<uint32_t*>(a.kcsz) +
                                 (static_cast<int64_t>(unit) * (a.capq / kKeyTile) + tile) * D);
}

size_t h2o_ws_bytes(int batch, int hkv, int T) {
  return static_cast<size_t>(batch) * hkv * (T > 0 ? T : 1) * sizeof(int32_t);
}

template <int D, int BITS, int NL, int IB, bool KT>
static hipError_t launch_dec(const H2OArgs& a, hipStream_t stream) {
  h2o_decode_kernel<D, BITS, NL, IB, KT><<<a.batch * a.hkv, 256, 0, stream>>>(a);
  return hipGetLastError();
}

template <int D, int BITS, int NL, int IB, bool KT>
static hipError_t launch_pre(const H2OArgs& a, hipStream_t stream) {
  const int T = a.len;
  int32_t* map = static_cast<int32_t*>(a.ws);
  h2o_prefill_select_kernel<<<a.batch * a.hkv, kSelThreads, 0, stream>>>(a, T, map);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || T == 0) return e;
  constexpr int RPB = 256 / (D / 8);
  const int64_t n_rows = static_cast<int64_t>(a.batch) * a.hkv * T;
  int64_t blocks = (n_rows + RPB - 1) / RPB;
  if (blocks > kScatterBlocks) blocks = kScatterBlocks;
  h2o_prefill_scatter_kernel<D, BITS, NL, IB, KT><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(a, T, map);
  e = hipGetLastError();
  if constexpr (KT) {
    const int tiles = (T - (a.cap16 - 1)) / kKeyTile;
    if (e == hipSuccess && tiles > 0)
      h2o_key_tile_kernel<D, BITS><<<static_cast<unsigned>(a.batch * a.hkv * tiles), 256, 0, stream>>>(a, T, tiles);
    e = hipGetLastError();
  }
  return e;
}

#define MIKV_H2O_DISPATCH(FN)                                                          \
  if (a.key_tile) {                                                                    \
    if (a.imp_bits != 16) return hipErrorInvalidValue;                                 \
    if (a.d == 128 && a.bits == 4 && a.group == 64) return FN<128, 4, 8, 16, true>(a, stream);  \
    if (a.d == 128 && a.bits == 4 && a.group == 128) return FN<128, 4, 16, 16, true>(a, stream); \
    if (a.d == 128 && a.bits == 2 && a.group == 64) return FN<128, 2, 8, 16, true>(a, stream);  \
    if (a.d == 128 && a.bits == 2 && a.group == 128) return FN<128, 2, 16, 16, true>(a, stream); \
    if (a.d == 64 && a.bits == 4 && a.group == 32) return FN<64, 4, 4, 16, true>(a, stream);    \
    if (a.d == 64 && a.bits == 4 && a.group == 64) return FN<64, 4, 8, 16, true>(a, stream);    \
    if (a.d == 64 && a.bits == 2 && a.group == 32) return FN<64, 2, 4, 16, true>(a, stream);    \
    if (a.d == 64 && a.bits == 2 && a.group == 64) return FN<64, 2, 8, 16, true>(a, stream);    \
    return hipErrorInvalidValue;                                                       \
  }                                                                                    \
  if (a.imp_bits == 16) {                                                              \
    if (a.d == 128 && a.bits == 4 && a.group == 64) return FN<128, 4, 8, 16, false>(a, stream);  \
    if (a.d == 128 && a.bits == 4 && a.group == 128) return FN<128, 4, 16, 16, false>(a, stream); \
    if (a.d == 128 && a.bits == 2 && a.group == 64) return FN<128, 2, 8, 16, false>(a, stream);  \
    if (a.d == 128 && a.bits == 2 && a.group == 128) return FN<128, 2, 16, 16, false>(a, stream); \
    if (a.d == 64 && a.bits == 4 && a.group == 32) return FN<64, 4, 4, 16, false>(a, stream);    \
    if (a.d == 64 && a.bits == 4 && a.group == 64) return FN<64, 4, 8, 16, false>(a, stream);    \
    if (a.d == 64 && a.bits == 2 && a.group == 32) return FN<64, 2, 4, 16, false>(a, stream);    \
    if (a.d == 64 && a.bits == 2 && a.group == 64) return FN<64, 2, 8, 16, false>(a, stream);    \
  } else if (a.group == a.d / 2) {                                                     \
    if (a.d == 128 && a.bits == 4 && a.imp_bits == 8) return FN<128, 4, 8, 8, false>(a, stream); \
    if (a.d == 128 && a.bits == 4 && a.imp_bits == 4) return FN<128, 4, 8, 4, false>(a, stream); \
    if (a.d == 128 && a.bits == 2 && a.imp_bits == 8) return FN<128, 2, 8, 8, false>(a, stream); \
    if (a.d == 128 && a.bits == 2 && a.imp_bits == 4) return FN<128, 2, 8, 4, false>(a, stream); \
    if (a.d == 64 && a.bits == 4 && a.imp_bits == 8) return FN<64, 4, 4, 8, false>(a, stream);   \
    if (a.d == 64 && a.bits == 4 && a.imp_bits == 4) return FN<64, 4, 4, 4, false>(a, stream);   \
    if (a.d == 64 && a.bits == 2 && a.imp_bits == 8) return FN<64, 2, 4, 8, false>(a, stream);   \
    if (a.d == 64 && a.bits == 2 && a.imp_bits == 4) return FN<64, 2, 4, 4, false>(a, stream);   \
  }                                                                                    \
  return hipErrorInvalidValue;

hipError_t launch_h2o_decode(const H2OArgs& a, hipStream_t stream) { MIKV_H2O_DISPATCH(launch_dec) }
hipError_t launch_h2o_prefill(const H2OArgs& a, hipStream_t stream) { MIKV_H2O_DISPATCH(launch_pre) }

}  // namespace mikv
