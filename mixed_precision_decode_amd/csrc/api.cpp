// C interface of the MiKV library: host-side validation and launches.
// Every function validates its arguments before anything is enqueued; see
// include/mikv.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.hpp"
#include "mikv.h"

using namespace mikv;

namespace {

bool supported_dims(int d, int group, int bits) {
  if (d != 64 && d != 128) return false;
  if (bits != 2 && bits != 4) return false;
  return group == d / 2 || group == d;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bits of the importance tier: 16 (fp16 rows; 0 means the same) or 8 / 4.
int imp_of(const mikv_dims* m) { return m->imp_bits == 0 ? 16 : m->imp_bits; }

mikv_status check_dims(const mikv_dims* m, bool need_tiers) {
  if (!m) return MIKV_ERR_NULL;
  if (m->batch < 1 || m->hq < 1 || m->hkv < 1 || m->d < 1) return MIKV_ERR_SHAPE;
  if (m->hq % m->hkv != 0) return MIKV_ERR_SHAPE;
  if (m->d != 64 && m->d != 128) return MIKV_ERR_UNSUPPORTED;
  if (need_tiers) {
    if (m->group < 1 || m->d % m->group != 0) return MIKV_ERR_SHAPE;
    if (m->bits != 2 && m->bits != 4) return MIKV_ERR_UNSUPPORTED;
    if (!supported_dims(m->d, m->group, m->bits)) return MIKV_ERR_UNSUPPORTED;
    if (m->cap16 < 1 || m->capq < 0) return MIKV_ERR_SHAPE;
    // a reduced-precision importance tier: 8- or 4-bit codes, groups of d/2
    const int ib = imp_of(m);
    if (ib != 16 && ib != 8 && ib != 4) return MIKV_ERR_UNSUPPORTED;
    if (ib != 16 && m->group != m->d / 2) return MIKV_ERR_UNSUPPORTED;
    // per-channel key tiles of 64 tokens: fp16 importance tier, whole tiles of slots
    if (m->key_tile != 0 && m->key_tile != kKeyTile) return MIKV_ERR_UNSUPPORTED;
    if (m->key_tile && ib != 16) return MIKV_ERR_UNSUPPORTED;
    if (m->key_tile && m->capq % kKeyTile != 0) return MIKV_ERR_SHAPE;
    // the decode kernels address one (sequence, kv head) tier with 32-bit byte offsets
    if (static_cast<int64_t>(m->capq) * m->d * m->bits / 8 >= (int64_t{1} << 31) ||
        static_cast<int64_t>(m->cap16) * m->d * ib / 8 >= (int64_t{1} << 31))
      return MIKV_ERR_SHAPE;
  }
  return MIKV_OK;
}

mikv_status check_cache(const mikv_cache* c, const mikv_dims* m) {
  const int imp_bits = imp_of(m);
  if (!c) return MIKV_ERR_NULL;
  if (!c->pos16 || !c->acc16 || !c->free16 || !c->kq || !c->vq || !c->vsz || !c->posq)
    return MIKV_ERR_NULL;
  if (!aligned16(c->kq) || !aligned16(c->vq)) return MIKV_ERR_SHAPE;
  if (m->key_tile) {
    if (!c->kcsz || !c->kbuf || !c->vbuf || !c->posbuf) return MIKV_ERR_NULL;
    if (!aligned16(c->kbuf) || !aligned16(c->vbuf)) return MIKV_ERR_SHAPE;
  } else if (!c->ksz) {
    return MIKV_ERR_NULL;
  }
  if (imp_bits == 16) {
    if (!c->k16 || !c->v16) return MIKV_ERR_NULL;
    if (!aligned16(c->k16) || !aligned16(c->v16)) return MIKV_ERR_SHAPE;
  } else {
    if (!c->kimp || !c->vimp || !c->kimpsz || !c->vimpsz) return MIKV_ERR_NULL;
    if (!aligned16(c->kimp) || !aligned16(c->vimp)) return MIKV_ERR_SHAPE;
  }
  return MIKV_OK;
}

void set_imp(DecodeArgs& a, const mikv_dims* m, const mikv_cache* c) {
  a.key_tile = m->key_tile;
  a.kcsz = c->kcsz; a.kbuf = c->kbuf; a.vbuf = c->vbuf;
  a.h2o.key_tile = m->key_tile;
  a.h2o.kcsz = reinterpret_cast<uint32_t*>(c->kcsz);
  a.h2o.kbuf = c->kbuf; a.h2o.vbuf = c->vbuf; a.h2o.posbuf = c->posbuf;
  a.imp_bits = imp_of(m);
  a.kimp = c->kimp; a.vimp = c->vimp; a.kimpsz = c->kimpsz; a.vimpsz = c->vimpsz;
  a.h2o.imp_bits = a.imp_bits;
  a.h2o.kimp = c->kimp; a.h2o.vimp = c->vimp;
  a.h2o.kimpsz = reinterpret_cast<uint32_t*>(c->kimpsz);
  a.h2o.vimpsz = reinterpret_cast<uint32_t*>(c->vimpsz);
}

void set_imp(H2OArgs& a, const mikv_dims* m, const mikv_cache* c) {
  a.key_tile = m->key_tile;
  a.kcsz = c->kcsz; a.kbuf = c->kbuf; a.vbuf = c->vbuf; a.posbuf = c->posbuf;
  a.imp_bits = imp_of(m);
  a.kimp = c->kimp; a.vimp = c->vimp; a.kimpsz = c->kimpsz; a.vimpsz = c->vimpsz;
}

mikv_status from_hip(hipError_t e) { return e == hipSuccess ? MIKV_OK : MIKV_ERR_HIP; }

}  // namespace

extern "C" {

const char* mikv_status_str(int s) {
  switch (s) {
    case MIKV_OK: return "ok";
    case MIKV_ERR_NULL: return "a required pointer is NULL";
    case MIKV_ERR_SHAPE: return "inconsistent sizes";
    case MIKV_ERR_UNSUPPORTED: return "unsupported head dim, bit width or group size";
    case MIKV_ERR_CAPACITY: return "low-bit tier capacity exceeded";
    case MIKV_ERR_WORKSPACE: return "workspace missing or too small";
    case MIKV_ERR_HIP: return "HIP call or kernel launch failed";
    case MIKV_ERR_SCRATCH: return "shape needs more than the library's fixed device scratch";
    default: return "unknown status";
  }
}

int mikv_abi_version(void) { return MIKV_ABI_VERSION; }

// ---------------------------------------------------------------- balancer
size_t mikv_balance_workspace(const mikv_dims* m, int32_t T) {
  if (check_dims(m, false) != MIKV_OK || T < 0) return 0;
  return balance_ws_bytes(m->batch, m->hkv, m->hq / m->hkv, m->d, T);
}

mikv_status mikv_balance_prefill(const mikv_dims* m, int32_t T, const uint16_t* q,
                                 const uint16_t* k, float* b, uint16_t* kb, void* ws,
                                 size_t ws_bytes, void* stream) {
  mikv_status st = check_dims(m, false);
  if (st != MIKV_OK) return st;
  if (T < 0) return MIKV_ERR_SHAPE;
  if (!b) return MIKV_ERR_NULL;
  if (T > 0 && (!q || !k)) return MIKV_ERR_NULL;
  if (T > 0 && (!aligned16(q) || !aligned16(k) || (kb && !aligned16(kb)))) return MIKV_ERR_SHAPE;
  const size_t need = balance_ws_bytes(m->batch, m->hkv, m->hq / m->hkv, m->d, T);
  if (need > 0 && (!ws || ws_bytes < need)) return MIKV_ERR_WORKSPACE;
  return from_hip(launch_balance(m->batch, m->hq, m->hkv, m->d, T, q, k, b, kb, ws,
                                 static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- prompt heavy-hitter scores
size_t mikv_prefill_scores_workspace(const mikv_dims* m, int32_t T) {
  if (check_dims(m, false) != MIKV_OK || T < 0) return 0;
  return prefill_scores_ws_bytes(m->batch, m->hq, T);
}

mikv_status mikv_prefill_scores(const mikv_dims* m, int32_t T, const uint16_t* q, const uint16_t* k,
                                float* acc0, void* ws, size_t ws_bytes, void* stream) {
  mikv_status st = check_dims(m, false);
  if (st != MIKV_OK) return st;
  if (T < 0) return MIKV_ERR_SHAPE;
  if (T == 0) return MIKV_OK;
  if (!q || !k || !acc0) return MIKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k)) return MIKV_ERR_SHAPE;
  // blocks of 256 rows per (sequence, head) must fit a 32-bit grid index
  if (static_cast<int64_t>(m->batch) * m->hq * ((T + 255) / 256) >= (int64_t{1} << 31)) return MIKV_ERR_SHAPE;
  const size_t need = prefill_scores_ws_bytes(m->batch, m->hq, T);
  if (!ws || ws_bytes < need) return MIKV_ERR_WORKSPACE;
  return from_hip(launch_prefill_scores(m->batch, m->hq, m->hkv, m->d, T, q, k, acc0, ws,
                                        static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- streaming-read probe
mikv_status mikv_read_probe(const void* p, size_t bytes, int32_t blocks, uint32_t* sink, void* stream) {
  if (bytes == 0) return MIKV_OK;
  if (!p || !sink) return MIKV_ERR_NULL;
  if (!aligned16(p) || bytes % 16 != 0 || blocks < 1) return MIKV_ERR_SHAPE;
  return from_hip(launch_read_probe(p, bytes, blocks, sink, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- quantize
mikv_status mikv_quantize_tokens(const uint16_t* x, const int32_t* rows, int64_t n_rows,
                                 int32_t d, int32_t group, int32_t bits, uint8_t* codes,
                                 uint16_t* sz, void* stream) {
  if (n_rows < 0 || d < 1 || group < 1) return MIKV_ERR_SHAPE;
  if (d % group != 0 || group % (8 / (bits == 2 ? 2 : 4)) != 0) return MIKV_ERR_SHAPE;
  if (!supported_dims(d, group, bits)) return MIKV_ERR_UNSUPPORTED;
  if (n_rows == 0) return MIKV_OK;
  if (!x || !codes || !sz) return MIKV_ERR_NULL;
  if (!aligned16(x)) return MIKV_ERR_SHAPE;
  return from_hip(launch_quantize_rows(x, rows, n_rows, d, group, bits, codes, sz,
                                       static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- decode attention
size_t mikv_decode_attn_workspace(const mikv_dims* m, int32_t max_len) {
  if (check_dims(m, true) != MIKV_OK) return 0;
  const int nq = max_len - m->cap16;
  if (nq < 0) return 0;
  return decode_ws_bound(m->batch, m->hq, m->hkv, m->d, m->bits, m->group, m->cap16, nq, imp_of(m),
                         m->key_tile);
}

static mikv_status decode_attn(const mikv_dims* m, const mikv_cache* c, int32_t len,
                               const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                               const float* b, float* o, float* p16, void* ws, size_t ws_bytes,
                               void* stream, void* ev_start, void* ev_stop) {
  mikv_status st = check_dims(m, true);
  if (st != MIKV_OK) return st;
  st = check_cache(c, m);
  if (st != MIKV_OK) return st;
  if (!q || !k_new || !v_new || !b || !o || !p16) return MIKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new)) return MIKV_ERR_SHAPE;
  const int nq = len - m->cap16;
  if (nq < 0) return MIKV_ERR_SHAPE;
  if (nq > m->capq) return MIKV_ERR_CAPACITY;
  const DecodePlan pl = decode_plan(m->batch, m->hkv, m->d, m->bits, m->group, m->hq / m->hkv,
                                    m->cap16, nq, imp_of(m), m->key_tile);
  const size_t need = decode_ws_bytes(m->batch, m->hq, m->hkv, m->d, m->cap16, pl);
  if (!ws || ws_bytes < need) return MIKV_ERR_WORKSPACE;
  DecodeArgs a;
  a.batch = m->batch; a.hq = m->hq; a.hkv = m->hkv; a.d = m->d; a.group = m->group;
  a.bits = m->bits; a.cap16 = m->cap16; a.capq = m->capq; a.len = len;
  a.q = q; a.k_new = k_new; a.v_new = v_new; a.b = b;
  a.k16 = c->k16; a.v16 = c->v16; a.pos16 = c->pos16; a.free16 = c->free16;
  a.kq = c->kq; a.vq = c->vq; a.ksz = c->ksz; a.vsz = c->vsz;
  a.o = o; a.p16 = p16; a.ws = ws;
  a.fuse_h2o = false;
  a.h2o = H2OView{};
  set_imp(a, m, c);
  a.ev_split_start = static_cast<hipEvent_t>(ev_start);
  a.ev_split_stop = static_cast<hipEvent_t>(ev_stop);
  return from_hip(launch_decode_attn(a, pl, static_cast<hipStream_t>(stream)));
}

mikv_status mikv_decode_attn(const mikv_dims* m, const mikv_cache* c, int32_t len,
                             const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                             const float* b, float* o, float* p16, void* ws, size_t ws_bytes,
                             void* stream) {
  return decode_attn(m, c, len, q, k_new, v_new, b, o, p16, ws, ws_bytes, stream, nullptr, nullptr);
}

mikv_status mikv_decode_attn_timed(const mikv_dims* m, const mikv_cache* c, int32_t len,
                                   const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                                   const float* b, float* o, float* p16, void* ws, size_t ws_bytes,
                                   void* stream, void* split_start, void* split_stop) {
  if (!split_start || !split_stop) return MIKV_ERR_NULL;
  return decode_attn(m, c, len, q, k_new, v_new, b, o, p16, ws, ws_bytes, stream, split_start,
                     split_stop);
}

}  // extern "C"

namespace {

// Host checks of a decode step; on success `plan` and `need` (workspace
// bytes for this length) are set.
mikv_status check_decode_step(const mikv_dims* m, const mikv_cache* c, int32_t len, int32_t recent,
                              int32_t heavy, const uint16_t* q, const uint16_t* k_new,
                              const uint16_t* v_new, const float* b, const float* o,
                              const float* p16, DecodePlan* plan, size_t* need) {
  mikv_status st = check_dims(m, true);
  if (st != MIKV_OK) return st;
  st = check_cache(c, m);
  if (st != MIKV_OK) return st;
  if (!q || !k_new || !v_new || !b || !o || !p16) return MIKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new)) return MIKV_ERR_SHAPE;
  if (recent < 0 || heavy < 0 || heavy + recent != m->cap16 - 1) return MIKV_ERR_SHAPE;
  const int nq = len - m->cap16;
  if (nq < 0) return MIKV_ERR_SHAPE;
  if (nq + 1 > m->capq) return MIKV_ERR_CAPACITY;  // the demotion adds one low-bit token
  *plan = decode_plan(m->batch, m->hkv, m->d, m->bits, m->group, m->hq / m->hkv, m->cap16, nq,
                      imp_of(m), m->key_tile);
  *need = decode_ws_bytes(m->batch, m->hq, m->hkv, m->d, m->cap16, *plan);
  return MIKV_OK;
}

// Launches of a checked decode step with workspace ws.
mikv_status launch_decode_step(const mikv_dims* m, const mikv_cache* c, int32_t len, int32_t recent,
                               int32_t heavy, const uint16_t* q, const uint16_t* k_new,
                               const uint16_t* v_new, const float* b, float* o, float* p16,
                               int32_t* demoted_pos, const DecodePlan& pl, void* ws, void* stream) {
  DecodeArgs a;
  a.batch = m->batch; a.hq = m->hq; a.hkv = m->hkv; a.d = m->d; a.group = m->group;
  a.bits = m->bits; a.cap16 = m->cap16; a.capq = m->capq; a.len = len;
  a.q = q; a.k_new = k_new; a.v_new = v_new; a.b = b;
  a.k16 = c->k16; a.v16 = c->v16; a.pos16 = c->pos16; a.free16 = c->free16;
  a.kq = c->kq; a.vq = c->vq; a.ksz = c->ksz; a.vsz = c->vsz;
  a.o = o; a.p16 = p16; a.ws = ws;
  // per-channel key tiles: the H2O step (buffer and tile flush) is its own launch
  a.fuse_h2o = m->key_tile == 0 && m->cap16 <= kFusedMaxCap16;
  a.ev_split_start = nullptr;
  a.ev_split_stop = nullptr;
  a.h2o = H2OView{};
  H2OView& v = a.h2o;
  v.cap16 = m->cap16; v.capq = m->capq; v.len = len; v.recent = recent;
  v.k16 = c->k16; v.v16 = c->v16; v.pos16 = c->pos16; v.acc16 = c->acc16; v.free16 = c->free16;
  v.kq = c->kq; v.vq = c->vq;
  v.ksz = reinterpret_cast<uint32_t*>(c->ksz);
  v.vsz = reinterpret_cast<uint32_t*>(c->vsz);
  v.posq = c->posq; v.demoted_pos = demoted_pos;
  set_imp(a, m, c);
  hipError_t e = launch_decode_attn(a, pl, static_cast<hipStream_t>(stream));
  if (e != hipSuccess || a.fuse_h2o) return from_hip(e);
  // large FP16 tiers: the H2O step runs as its own launch
  H2OArgs h = {};
  h.batch = m->batch; h.hkv = m->hkv; h.d = m->d; h.group = m->group; h.bits = m->bits;
  h.cap16 = m->cap16; h.capq = m->capq; h.len = len; h.recent = recent; h.heavy = heavy;
  h.k16 = c->k16; h.v16 = c->v16; h.pos16 = c->pos16; h.acc16 = c->acc16; h.free16 = c->free16;
  h.kq = c->kq; h.vq = c->vq; h.ksz = c->ksz; h.vsz = c->vsz; h.posq = c->posq;
  h.p16 = p16; h.demoted_pos = demoted_pos;
  set_imp(h, m, c);
  return from_hip(launch_h2o_decode(h, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

mikv_status mikv_decode_step(const mikv_dims* m, const mikv_cache* c, int32_t len, int32_t recent,
                             int32_t heavy, const uint16_t* q, const uint16_t* k_new,
                             const uint16_t* v_new, const float* b, float* o, float* p16,
                             int32_t* demoted_pos, void* ws, size_t ws_bytes, void* stream) {
  DecodePlan pl;
  size_t need = 0;
  const mikv_status st = check_decode_step(m, c, len, recent, heavy, q, k_new, v_new, b, o, p16, &pl, &need);
  if (st != MIKV_OK) return st;
  if (!ws || ws_bytes < need) return MIKV_ERR_WORKSPACE;
  return launch_decode_step(m, c, len, recent, heavy, q, k_new, v_new, b, o, p16, demoted_pos, pl, ws,
                            stream);
}

size_t mikv_decode_step_noalloc_limit(void) { return kStaticScratchBytes; }

mikv_status mikv_decode_step_noalloc(const mikv_dims* m, const mikv_cache* c, int32_t len,
                                     int32_t recent, int32_t heavy, const uint16_t* q,
                                     const uint16_t* k_new, const uint16_t* v_new, const float* b,
                                     float* o, float* p16, int32_t* demoted_pos, void* stream) {
  DecodePlan pl;
  size_t need = 0;
  const mikv_status st = check_decode_step(m, c, len, recent, heavy, q, k_new, v_new, b, o, p16, &pl, &need);
  if (st != MIKV_OK) return st;
  if (need > kStaticScratchBytes) return MIKV_ERR_SCRATCH;
  void* ws = nullptr;
  if (static_scratch_ptr(&ws) != hipSuccess || !ws) return MIKV_ERR_HIP;
  return launch_decode_step(m, c, len, recent, heavy, q, k_new, v_new, b, o, p16, demoted_pos, pl, ws,
                            stream);
}

// ---------------------------------------------------------------- H2O
size_t mikv_h2o_workspace(const mikv_dims* m, int32_t max_T) {
  if (check_dims(m, true) != MIKV_OK || max_T < 0) return 0;
  return h2o_ws_bytes(m->batch, m->hkv, max_T);
}

mikv_status mikv_h2o_update_select(const mikv_dims* m, const mikv_cache* c, int32_t len,
                                   int32_t recent, int32_t heavy, const float* p16,
                                   const mikv_prefill_src* src, int32_t* demoted_pos, void* ws,
                                   size_t ws_bytes, void* stream) {
  mikv_status st = check_dims(m, true);
  if (st != MIKV_OK) return st;
  st = check_cache(c, m);
  if (st != MIKV_OK) return st;
  if ((p16 == nullptr) == (src == nullptr)) return MIKV_ERR_NULL;
  if (recent < 0 || heavy < 0 || heavy + recent != m->cap16 - 1) return MIKV_ERR_SHAPE;
  H2OArgs a = {};
  a.batch = m->batch; a.hkv = m->hkv; a.d = m->d; a.group = m->group; a.bits = m->bits;
  a.cap16 = m->cap16; a.capq = m->capq; a.len = len; a.recent = recent; a.heavy = heavy;
  a.k16 = c->k16; a.v16 = c->v16; a.pos16 = c->pos16; a.acc16 = c->acc16; a.free16 = c->free16;
  a.kq = c->kq; a.vq = c->vq; a.ksz = c->ksz; a.vsz = c->vsz; a.posq = c->posq;
  set_imp(a, m, c);
  const int B = m->cap16 - 1;
  if (p16) {
    // decode: the low-bit tier grows to len - B tokens
    if (len - m->cap16 < 0) return MIKV_ERR_SHAPE;
    if (len - B > m->capq) return MIKV_ERR_CAPACITY;
    a.p16 = p16;
    a.demoted_pos = demoted_pos;
    return from_hip(launch_h2o_decode(a, static_cast<hipStream_t>(stream)));
  }
  if (src->T != len || len < B) return MIKV_ERR_SHAPE;
  if (len > 0 && (!src->k || !src->v || !src->acc0)) return MIKV_ERR_NULL;
  if (len > 0 && (!aligned16(src->k) || !aligned16(src->v) || (src->b && !aligned16(src->b))))
    return MIKV_ERR_SHAPE;
  if (len - B > m->capq) return MIKV_ERR_CAPACITY;
  const size_t need = h2o_ws_bytes(m->batch, m->hkv, len);
  if (!ws || ws_bytes < need) return MIKV_ERR_WORKSPACE;
  a.src_k = src->k; a.src_v = src->v; a.src_acc0 = src->acc0; a.src_b = src->b;
  a.ws = ws;
  return from_hip(launch_h2o_prefill(a, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- output perturbation
size_t mikv_perturbation_workspace(int32_t H, int32_t T, int32_t d, int32_t hidden) {
  if (H < 1 || T < 1 || (d != 64 && d != 128) || hidden < 1) return 0;
  return perturbation_ws_bytes(H, T, d, hidden);
}

mikv_status mikv_output_perturbation(const uint16_t* q, const uint16_t* K, const uint16_t* V,
                                     const uint16_t* W_O, const int32_t* keep, int32_t n_keep,
                                     const float* o_hat, int32_t H, int32_t T, int32_t d, int32_t hidden,
                                     float* o, float* delta, float* L_head, float* L_proj, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (!q || !K || !V || !W_O || !L_head || !L_proj) return MIKV_ERR_NULL;
  if ((keep == nullptr) == (o_hat == nullptr)) return MIKV_ERR_NULL;
  if (H < 1 || T < 1 || hidden < 1) return MIKV_ERR_SHAPE;
  if (d != 64 && d != 128) return MIKV_ERR_UNSUPPORTED;
  if (keep && (n_keep < 1 || n_keep > T)) return MIKV_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(K) || !aligned16(V)) return MIKV_ERR_SHAPE;
  // one head's rows (of K and V, and of W_O) are addressed with 32-bit byte offsets
  if (static_cast<int64_t>(T) * d * 2 >= (int64_t{1} << 31)) return MIKV_ERR_SHAPE;
  if (static_cast<int64_t>(hidden) * d * 2 + 1024 >= (int64_t{1} << 31)) return MIKV_ERR_SHAPE;
  const size_t need = perturbation_ws_bytes(H, T, d, hidden);
  if (!ws || ws_bytes < need) return MIKV_ERR_WORKSPACE;
  return from_hip(launch_perturbation(q, K, V, W_O, keep, n_keep, o_hat, H, T, d, hidden, o, delta, L_head,
                                      L_proj, ws, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- CriticalKV
size_t mikv_criticalkv_workspace(int32_t H, int32_t T, int32_t d, int32_t hidden) {
  if (H < 1 || T < 1 || d != 128 || hidden < 128 || hidden % 128 != 0) return 0;
  return criticalkv_ws_bytes(H, T, d, hidden);
}

mikv_status mikv_criticalkv_select(const float* A, const uint16_t* V, const uint16_t* W_O,
                                   int32_t H, int32_t T, int32_t d, int32_t hidden,
                                   int32_t budget, double alpha, int32_t* idx, float* score2,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (!A || !V || !W_O || !idx) return MIKV_ERR_NULL;
  if (H < 1 || T < 1 || hidden < 1) return MIKV_ERR_SHAPE;
  if (d != 128) return MIKV_ERR_UNSUPPORTED;
  if (hidden % 128 != 0) return MIKV_ERR_UNSUPPORTED;
  if (budget < 1 || budget > T) return MIKV_ERR_SHAPE;
  if (!(alpha >= 0.0 && alpha <= 1.0)) return MIKV_ERR_SHAPE;
  if (!aligned16(V) || !aligned16(W_O)) return MIKV_ERR_SHAPE;
  const size_t need = criticalkv_ws_bytes(H, T, d, hidden);
  if (!ws || ws_bytes < need) return MIKV_ERR_WORKSPACE;
  const int b1 = static_cast<int>(std::floor(alpha * budget));
  const int b2 = budget - b1;
  return from_hip(launch_criticalkv(A, V, W_O, H, T, d, hidden, b1, b2, idx, score2, ws,
                                    static_cast<hipStream_t>(stream)));
}

}  // extern "C"
