// Host-side launchers of the MiKV kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "h2o_common.hpp"

namespace mikv {

hipError_t launch_quantize_rows(const uint16_t* x, const int32_t* rows, int64_t n_rows, int d,
                                int group, int bits, uint8_t* codes, uint16_t* sz,
                                hipStream_t stream);

// Channel balancer: partial maxima per token chunk, then finalize; optional kb.
size_t balance_ws_bytes(int batch, int hkv, int rep, int d, int T);
hipError_t launch_balance(int batch, int hq, int hkv, int d, int T, const uint16_t* q,
                          const uint16_t* k, float* b, uint16_t* kb, void* ws,
                          hipStream_t stream);

struct DecodePlan {
  int C16, Cq;     // tokens per split in the FP16 / low-bit tier
  int S16, Sq;     // splits per tier
  int RT;          // query heads per block
  int tiles;       // rep / RT
  int f16_first;   // 1: FP16-tier splits take the first block indices (else the low-bit splits do)
  int nq;          // low-bit tokens attended (per-channel key tiles: whole tiles only)
  int nb, Sb;      // per-channel key tiles: buffered fp16 pairs and their splits (0 or 1)
  int key_tile;    // 0: per-token keys; 64: per-channel key tiles
};
// nr = retained tokens when the step starts (len - cap16)
DecodePlan decode_plan(int batch, int hkv, int d, int bits, int group, int rep, int cap16, int nr,
                       int imp_bits, int key_tile);
size_t decode_ws_bytes(int batch, int hq, int hkv, int d, int cap16, const DecodePlan& plan);
// workspace that serves every length up to nr_max retained tokens
size_t decode_ws_bound(int batch, int hq, int hkv, int d, int bits, int group, int cap16, int nr_max,
                       int imp_bits, int key_tile);

struct DecodeArgs {
  int batch, hq, hkv, d, group, bits, cap16, capq, len;
  int imp_bits;  // 16: fp16 importance tier (k16, v16); 8 or 4: codes (kimp, vimp)
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
  const uint16_t* ksz;
  const uint16_t* vsz;
  uint8_t* kimp;
  uint8_t* vimp;
  uint16_t* kimpsz;
  uint16_t* vimpsz;
  float* o;
  float* p16;
  void* ws;
  // per-channel key tiles (key_tile = 64)
  int key_tile;
  const uint16_t* kcsz;
  const uint16_t* kbuf;
  const uint16_t* vbuf;
  // fused decode step: the merge kernel also runs the H2O update, re-select
  // and demotion (fuse_h2o = true; h2o holds the cache views it writes)
  bool fuse_h2o;
  H2OView h2o;
  // optional hipEvent_t pair that records the split kernel's own start and
  // end (hipExtLaunchKernel); both null for an ordinary launch
  hipEvent_t ev_split_start, ev_split_stop;
};
hipError_t launch_decode_attn(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);
// largest FP16 tier the fused merge handles (slots held in registers)
constexpr int kFusedMaxCap16 = 16 * 256;

// Fixed device scratch of mikv_decode_step_noalloc (16 MiB per device).
constexpr size_t kStaticScratchBytes = size_t{16} << 20;
hipError_t static_scratch_ptr(void** ptr);

struct H2OArgs {
  int batch, hkv, d, group, bits, cap16, capq, len, recent, heavy;
  int imp_bits;  // 16: fp16 importance tier; 8 or 4: codes (kimp, vimp)
  uint8_t* kimp;
  uint8_t* vimp;
  uint16_t* kimpsz;
  uint16_t* vimpsz;
  uint16_t* k16;
  uint16_t* v16;
  int32_t* pos16;
  float* acc16;
  int32_t* free16;
  uint8_t* kq;
  uint8_t* vq;
  uint16_t* ksz;
  uint16_t* vsz;
  int32_t* posq;
  const float* p16;
  int32_t* demoted_pos;
  // per-channel key tiles (key_tile = 64; 0 = per-token keys)
  int key_tile;
  uint16_t* kcsz;
  uint16_t* kbuf;
  uint16_t* vbuf;
  int32_t* posbuf;
  // prefill
  const uint16_t* src_k;
  const uint16_t* src_v;
  const float* src_acc0;
  const float* src_b;
  void* ws;
};
size_t h2o_ws_bytes(int batch, int hkv, int T);
hipError_t launch_h2o_decode(const H2OArgs& a, hipStream_t stream);
hipError_t launch_h2o_prefill(const H2OArgs& a, hipStream_t stream);

// Prompt heavy-hitter scores: per-query softmax statistics, then column sums.
size_t prefill_scores_ws_bytes(int batch, int hq, int T);
hipError_t launch_prefill_scores(int batch, int hq, int hkv, int d, int T, const uint16_t* q,
                                 const uint16_t* k, float* acc0, void* ws, hipStream_t stream);

// Streaming-read probe (measurement): reads `bytes` (a multiple of 16) of p.
hipError_t launch_read_probe(const void* p, size_t bytes, int blocks, uint32_t* sink, hipStream_t stream);

// Output-perturbation diagnostic.
int perturbation_splits(int H, int T);
size_t perturbation_ws_bytes(int H, int T, int d, int hidden);
hipError_t launch_perturbation(const uint16_t* q, const uint16_t* K, const uint16_t* V, const uint16_t* W,
                               const int32_t* keep, int n_keep, const float* o_hat, int H, int T, int d,
                               int hidden, float* o, float* delta_out, float* L_head, float* L_proj,
                               void* ws, hipStream_t stream);

size_t criticalkv_ws_bytes(int H, int T, int d, int hidden);
hipError_t launch_criticalkv(const float* A, const uint16_t* V, const uint16_t* W, int H, int T,
                             int d, int hidden, int b1, int b2, int32_t* idx, float* score2,
                             void* ws, hipStream_t stream);

}  // namespace mikv
