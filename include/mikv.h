/*
 * mikv.h - C interface of the MiKV mixed-precision KV-cache path for
 * AMD Instinct MI355X (gfx950).
 *
 * Method sources (cited by page title and section):
 *   [velog notes]      velog.io post "No Token Left Behind: Reliable KV Cache
 *                      Compression via Importance-Aware Mixed Precision
 *                      Quantization" (reader's notes on arXiv 2402.18096).
 *   [paperlayer]       paperlayer.ai source-linked summary of arXiv
 *                      2402.18096v1, "No Token Left Behind ...".
 *   [gist CriticalKV]  gist.science technical summary of arXiv 2502.03805
 *                      (CriticalKV).
 *
 * Conventions for every entry point
 *   - fp16 tensors are passed as uint16_t bit patterns (IEEE binary16).
 *   - Every tensor pointer is DEVICE memory owned by the caller; the library
 *     never allocates, frees or synchronises. Its only global state is a
 *     per-process cache of launch facts (each device's compute-unit count
 *     and the kernels' occupancy), filled on first use with relaxed atomics
 *     and never changed afterwards, so concurrent calls from several host
 *     threads are safe. Tensors are dense row-major in the index order
 *     written next to them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls validate their arguments on the host, enqueue kernels on
 *     `stream` and return at once. On a validation failure nothing is
 *     enqueued and the status says why. A failed launch returns
 *     MIKV_ERR_HIP. Faults inside kernels surface at the caller's next
 *     synchronisation. No C++ exception crosses this interface.
 *   - Supported shapes: head dim d in {64, 128}; bits in {2, 4}; group in
 *     {d/2, d} (d/2 is the method's setting); hq a multiple of hkv;
 *     imp_bits in {16 (or 0), 8, 4}, 8 and 4 with group d/2 only
 *     (MIKV_ERR_UNSUPPORTED otherwise).
 *   - Inputs must be finite; non-finite values give unspecified results.
 *
 * Two-tier cache (mikv_cache), per sequence n and kv head g:
 *   FP16 "importance" tier, cap16 slots:
 *     k16, v16 [batch][hkv][cap16][d] fp16   balanced keys k*b, values
 *     pos16    [batch][hkv][cap16]    int32  token position of the slot
 *     acc16    [batch][hkv][cap16]    fp32   H2O accumulated attention
 *     free16   [batch][hkv]           int32  the one free slot
 *   Low-bit "retention" tier, capq slots, filled in order 0,1,2,...:
 *     kq, vq   [batch][hkv][capq][d*bits/8] uint8  packed codes
 *     ksz, vsz [batch][hkv][capq][d/group][2] fp16 (scale, zero) per group
 *     posq     [batch][hkv][capq]     int32  token position of the slot
 *   Code packing: code of channel (8/bits)*j + m sits in bits
 *   [bits*m, bits*m+bits) of byte j. Dequantized value = code*scale + zero.
 * Reduced-precision importance tier ([velog notes] Key contributions 3);
 * [paperlayer] section 3.3: the importance cache itself quantized, e.g.
 * INT4 or INT8 over a 2-bit retention cache), selected by dims.imp_bits:
 *   imp_bits 16 (or 0): the FP16 tier above (k16, v16).
 *   imp_bits 8 or 4: k16 and v16 are unused (may be NULL) and the tier holds
 *     kimp, vimp [batch][hkv][cap16][d*imp_bits/8] uint8 codes and
 *     kimpsz, vimpsz [batch][hkv][cap16][d/group][2] fp16 (scale, zero),
 *     packed like the low-bit tier; requires group == d/2. A new token is
 *     quantized as it is appended; a demoted token is re-quantized to `bits`
 *     from its codes rebuilt as the fp16 row fp16(code*scale + zero).
 *   Grouping pairs by precision is allowed because attention is invariant
 *   under jointly permuting KV pairs ([velog notes] section 3.4).
 * Per-channel key quantization ([velog notes] the per-channel alternative
 * and its appendix C summary; [paperlayer] appendix C: retained keys
 * quantized per channel with groups of 64 tokens, which needs a buffer
 * for pairs until enough have gathered), selected by dims.key_tile = 64
 * (requires imp_bits 16 and capq a multiple of 64):
 *   kq      [batch][hkv][capq][d*bits/8] uint8: tiles of 64 consecutive
 *           slots, packed token-major as above; ksz is unused (may be NULL)
 *   kcsz    [batch][hkv][capq/64][d][2] fp16 (scale, zero) per tile and
 *           channel: the per-token rule run along the tile's 64 tokens
 *   vq, vsz values per token, as above
 *   kbuf, vbuf [batch][hkv][64][d] fp16, posbuf [batch][hkv][64] int32:
 *           pairs that left the importance tier and wait for a tile.
 *   A cache whose retained tier has taken D tokens holds 64*floor(D/64) of
 *   them in tiles (slots 0..) and the other D mod 64 in buffer rows
 *   0..D mod 64 - 1, both in the order they were demoted; buffered pairs
 *   are attended to in fp16. The demotion that fills the buffer turns it
 *   into the next tile (keys per channel, values per token).
 *   With B = cap16 - 1 important tokens and a current length N (new token
 *   included), the low-bit tier holds N - 1 - B tokens when a decode step
 *   starts and N - B after it.
 */
#ifndef MIKV_H
#define MIKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MIKV_ABI_VERSION 4

typedef enum {
  MIKV_OK = 0,
  MIKV_ERR_NULL = 1,        /* a required pointer is NULL                   */
  MIKV_ERR_SHAPE = 2,       /* sizes inconsistent with each other           */
  MIKV_ERR_UNSUPPORTED = 3, /* d, bits or group outside the supported set   */
  MIKV_ERR_CAPACITY = 4,    /* the low-bit tier would exceed capq slots     */
  MIKV_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required      */
  MIKV_ERR_HIP = 6,         /* a HIP call or kernel launch failed           */
  MIKV_ERR_SCRATCH = 7      /* shape needs more than the fixed device
                               scratch of mikv_decode_step_noalloc          */
} mikv_status;

/* Static English text for a status value (never NULL). */
const char* mikv_status_str(int status);

/* MIKV_ABI_VERSION of the built library. */
int mikv_abi_version(void);

typedef struct {
  int32_t batch; /* sequences n                                            */
  int32_t hq;    /* query heads                                            */
  int32_t hkv;   /* kv heads; query head h uses kv head h / (hq/hkv)       */
  int32_t d;     /* head dim, 64 or 128                                    */
  int32_t group; /* channels per quantization group: d/2 or d              */
  int32_t bits;  /* low-bit code width, 4 or 2                             */
  int32_t cap16; /* FP16-tier slots per (n, g) = B + 1                     */
  int32_t capq;  /* low-bit-tier slots per (n, g)                          */
  int32_t imp_bits; /* importance tier: 16 or 0 = fp16 rows; 8 or 4 = codes */
  int32_t key_tile; /* 0: per-token keys; 64: per-channel keys over tiles of
                       64 tokens with an fp16 token buffer (see above)     */
} mikv_dims;

typedef struct {
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
  uint8_t* kimp;    /* importance tier as codes (imp_bits 8 or 4), else NULL */
  uint8_t* vimp;
  uint16_t* kimpsz;
  uint16_t* vimpsz;
  uint16_t* kcsz;   /* per-channel key tiles (key_tile 64), else NULL     */
  uint16_t* kbuf;
  uint16_t* vbuf;
  int32_t* posbuf;
} mikv_cache;

/*
 * Channel balancer ([velog notes] Key contributions 2), balancer equation
 * and k-hat equation; [paperlayer] section 3.2).
 *   b[n][g][c] = sqrt( max_{h in group g, t < T} |q[n][h][t][c]|
 *                      / max_{t < T} |k[n][g][t][c]| )      (fp32 IEEE ops)
 *   b = 1 where either maximum is 0 (also when T == 0).
 *   kb[n][g][t][c] = fp16_rne( fp32(k) * b[n][g][c] ), written if kb != NULL.
 * q  [batch][hq][T][d] fp16, k [batch][hkv][T][d] fp16 (inputs).
 * b  [batch][hkv][d] fp32 (output), kb [batch][hkv][T][d] fp16 (output).
 * ws: workspace of mikv_balance_workspace(dims, T) bytes (any contents).
 * dims->group, bits, cap16, capq are not used.
 */
size_t mikv_balance_workspace(const mikv_dims* dims, int32_t T);
mikv_status mikv_balance_prefill(const mikv_dims* dims, int32_t T,
                                 const uint16_t* q, const uint16_t* k,
                                 float* b, uint16_t* kb,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * Per-token asymmetric quantization with groups ([velog notes] Key
 * contributions 1): per-token asymmetric (LLM-QAT style); Key contributions
 * 2), additional notes: group = half the head dim; [paperlayer] section 3.2).
 * For output row r, source row x[rows ? rows[r] : r] and each group of
 * `group` contiguous channels:
 *   scale = fp16_rne((fp32(max) - fp32(min)) / (2^bits - 1)), zero = min;
 *   code  = clamp(rint_half_even((fp32(x) - fp32(zero)) / fp32(scale)),
 *                 0, 2^bits - 1), all codes 0 when scale == 0;
 *   a zero scale or zero point is stored as +0.
 * x [*][d] fp16; rows [n_rows] int32 or NULL; codes [n_rows][d*bits/8] uint8
 * and sz [n_rows][d/group][2] fp16 (outputs). n_rows == 0 enqueues nothing.
 * The caller guarantees 0 <= rows[r] < (rows of x).
 */
mikv_status mikv_quantize_tokens(const uint16_t* x, const int32_t* rows,
                                 int64_t n_rows, int32_t d, int32_t group,
                                 int32_t bits, uint8_t* codes, uint16_t* sz,
                                 void* stream);

/*
 * One decode step of mixed-precision attention ([velog notes] section 3.4
 * and [paperlayer] section 3.4: decode attention is a memory-bound batched
 * matrix-vector product over a precision-grouped cache whose keys and values
 * are low precision while the query and the attention map stay floating
 * point; [velog notes] Key contributions 2): q-hat = q / b).
 *   1. Append: the new token (position len-1) goes into FP16 slot
 *      free16[n][g]: k16 = fp16_rne(fp32(k_new) * b), v16 = v_new,
 *      pos16 = len-1 (acc16 and free16 are left to mikv_h2o_update_select).
 *   2. For each query head h of kv head g, q-hat = fp32(q) / b and
 *      s_i = q-hat . k~_i / sqrt(d) over the cap16 FP16-tier tokens
 *      (k~ = k16) and the len - cap16 low-bit tokens (k~ = code*scale+zero);
 *      p = softmax(s) over both tiers; o[n][h] = sum_i p_i v~_i.
 *      The kernels form q-hat as fp32(q) times the hardware reciprocal of b
 *      (within 1 ulp of the quotient) with 1/sqrt(d) folded in; scores only
 *      enter outputs that are specified to a tolerance.
 *   3. p16[n][g][slot] = sum over the query heads of group g of p at that
 *      FP16 slot (input of the H2O accumulation).
 *      Per-channel key tiles: the len - cap16 retained tokens are the
 *      whole tiles (k~[c] = code*scale[c] + zero[c] of the tile) and the
 *      (len - cap16) mod 64 buffered pairs (k~ = kbuf, v~ = vbuf in fp16).
 * Precondition: the low-bit tier holds len - cap16 tokens (slots
 * 0..len-cap16-1); every FP16 slot other than free16 is occupied. The free
 * slot's stale K/V rows are read and masked, so they must hold finite fp16
 * values (the prefill build zeroes them; afterwards they hold the token the
 * last step demoted).
 * q [batch][hq][d] fp16, k_new/v_new [batch][hkv][d] fp16, b [batch][hkv][d]
 * fp32 (inputs); o [batch][hq][d] fp32, p16 [batch][hkv][cap16] fp32
 * (outputs). Accumulation is fp32.
 * ws: mikv_decode_attn_workspace(dims, max_len) bytes (any contents), valid
 * for any len <= max_len; it holds the per-split partial results between the
 * two kernels of the call. One workspace serves one call at a time.
 * Errors: len - cap16 < 0 -> MIKV_ERR_SHAPE; len - cap16 > capq ->
 * MIKV_ERR_CAPACITY; a per-(sequence, kv head) tier of 2^31 bytes or more
 * (capq*d*bits/8 or cap16*2*d) -> MIKV_ERR_SHAPE (the kernels address a tier
 * with 32-bit offsets); key_tile not 0 or 64, or 64 with imp_bits 8 or 4
 * -> MIKV_ERR_UNSUPPORTED; key_tile 64 with capq not a multiple of 64 ->
 * MIKV_ERR_SHAPE; key_tile 64 with kcsz, kbuf, vbuf or posbuf NULL ->
 * MIKV_ERR_NULL, kbuf or vbuf not 16-byte aligned -> MIKV_ERR_SHAPE.
 */
size_t mikv_decode_attn_workspace(const mikv_dims* dims, int32_t max_len);
mikv_status mikv_decode_attn(const mikv_dims* dims, const mikv_cache* cache,
                             int32_t len, const uint16_t* q,
                             const uint16_t* k_new, const uint16_t* v_new,
                             const float* b, float* o, float* p16,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * mikv_decode_attn with the duration of its first kernel measured: the
 * same computation, arguments, outputs and errors, and in addition the
 * caller's events split_start and split_stop (hipEvent_t passed as void*,
 * created with timing enabled, owned by the caller) receive the start and
 * end timestamps of the split kernel, which streams both cache tiers and
 * moves nearly all of the call's bytes. hipEventElapsedTime(split_start,
 * split_stop) is then that kernel's duration alone, without launch gaps.
 * The events are recorded through hipExtLaunchKernel on `stream`.
 * Errors: as mikv_decode_attn; a NULL event -> MIKV_ERR_NULL.
 */
mikv_status mikv_decode_attn_timed(const mikv_dims* dims, const mikv_cache* cache,
                                   int32_t len, const uint16_t* q,
                                   const uint16_t* k_new, const uint16_t* v_new,
                                   const float* b, float* o, float* p16,
                                   void* ws, size_t ws_bytes, void* stream,
                                   void* split_start, void* split_stop);

/*
 * Prompt heavy-hitter scores acc0 (input of the prefill build of
 * mikv_h2o_update_select): the attention each prompt token has accumulated
 * during the prompt ([paperlayer] section 5 and [velog notes] Key
 * contributions 1): important tokens are the heavy hitters of accumulated
 * attention, H2O). For query head h of kv head g and query position i,
 * P[i][t] = softmax over t <= i of q[n][h][i] . k[n][g][t] / sqrt(d)
 * (causal); acc0[n][g][t] = sum over the group's query heads h and the
 * queries i >= t of P[i][t]. Each row of P sums to 1, so the scores of a
 * (sequence, kv head) sum to (hq/hkv) * T.
 * q [batch][hq][T][d], k [batch][hkv][T][d] fp16 as given to the model's
 * attention (not balanced: the balancer leaves q . k unchanged);
 * acc0 [batch][hkv][T] fp32 (output). Scores on matrix cores (fp16 inputs,
 * fp32 accumulation), softmax and sums in fp32.
 * ws: mikv_prefill_scores_workspace(dims, T) bytes (any contents): the
 * log-sum-exp of every query row between the two kernels.
 * Only batch, hq, hkv and d of dims are used. T == 0 enqueues nothing.
 * Errors: NULL pointer -> MIKV_ERR_NULL; q or k not 16-byte aligned, T < 0
 * -> MIKV_ERR_SHAPE; d not in {64, 128} -> MIKV_ERR_UNSUPPORTED; workspace
 * too small -> MIKV_ERR_WORKSPACE.
 */
size_t mikv_prefill_scores_workspace(const mikv_dims* dims, int32_t T);
mikv_status mikv_prefill_scores(const mikv_dims* dims, int32_t T,
                                const uint16_t* q, const uint16_t* k,
                                float* acc0, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * Measurement helper, not a step of the method: a plain streaming read of
 * `bytes` of device memory at p (16-byte nontemporal loads, `blocks`
 * workgroups of 256 threads, each reading one contiguous chunk), so that the
 * HBM bandwidth of the decode kernels can be compared with what a kernel
 * that only reads reaches on the same device. sink [blocks] uint32 receives
 * one word per block (an XOR of the data, which keeps the loads live).
 * bytes == 0 enqueues nothing.
 * Errors: NULL p or sink -> MIKV_ERR_NULL; p not 16-byte aligned, bytes not
 * a multiple of 16, blocks < 1 -> MIKV_ERR_SHAPE.
 */
mikv_status mikv_read_probe(const void* p, size_t bytes, int32_t blocks,
                            uint32_t* sink, void* stream);

/*
 * Source of the prefill build of mikv_h2o_update_select.
 *   k    [batch][hkv][T][d] fp16  prompt keys (multiplied by b when b != NULL,
 *                                 exactly as mikv_balance_prefill's kb)
 *   v    [batch][hkv][T][d] fp16  prompt values
 *   acc0 [batch][hkv][T]    fp32  accumulated attention of the prompt (>= 0)
 *   b    [batch][hkv][d]    fp32  balancer or NULL (keys used as given)
 */
typedef struct {
  const uint16_t* k;
  const uint16_t* v;
  const float* acc0;
  const float* b;
  int32_t T;
} mikv_prefill_src;

/*
 * Heavy-hitter bookkeeping, important-set re-selection and demotion
 * ([velog notes] one-line summary and Key contributions 1): tokens an
 * importance-based (H2O) eviction would drop are kept as low-bit codes;
 * [paperlayer] section 5: heavy hitters plus local tokens). The ranking key
 * is (accumulated attention descending, token position ascending). The
 * recent window is the `recent` newest positions. Requires
 * heavy + recent == cap16 - 1 (= B).
 *
 * Decode mode (p16 != NULL, src == NULL), after mikv_decode_attn at the
 * same len:
 *   acc16[slot] = (slot == free16 ? 0 : acc16[slot]) + p16[slot];
 *   candidates = FP16 slots with pos16 < len - recent (heavy + 1 of them);
 *   the candidate outside the top-`heavy` is quantized (as in
 *   mikv_quantize_tokens, keys and values) into low-bit slot len - cap16,
 *   its position copied to posq, and free16 set to its slot.
 *   demoted_pos[n][g] (optional) receives its position.
 *   Per-channel key tiles: the candidate's fp16 key and value rows go to
 *   buffer row (len - cap16) mod 64 (position to posbuf); when that is row
 *   63 the buffer becomes tile (len - cap16) / 64.
 * Prefill mode (p16 == NULL, src != NULL, len == src->T):
 *   important = positions >= T - recent plus the top-`heavy` positions of
 *   [0, T - recent) by (acc0 desc, position asc); they fill FP16 slots
 *   0..B-1 in ascending position with acc16 = acc0, free16 = B (its K/V
 *   rows zeroed, pos16 = -1, acc16 = 0); the other T - B positions are
 *   quantized into low-bit slots 0..T-B-1 in ascending position
 *   (per-channel key tiles: the first 64*floor((T-B)/64) of them fill
 *   tiles, the last (T-B) mod 64 go to the buffer as fp16).
 *   demoted_pos is ignored.
 * ws: mikv_h2o_workspace(dims, max_T) bytes (any contents; decode mode
 * needs none and accepts ws == NULL).
 * Errors: T < B -> MIKV_ERR_SHAPE; src->k, src->v or a non-NULL src->b not
 * 16-byte aligned -> MIKV_ERR_SHAPE; low-bit tier overflow ->
 * MIKV_ERR_CAPACITY.
 */
size_t mikv_h2o_workspace(const mikv_dims* dims, int32_t max_T);
mikv_status mikv_h2o_update_select(const mikv_dims* dims,
                                   const mikv_cache* cache, int32_t len,
                                   int32_t recent, int32_t heavy,
                                   const float* p16,
                                   const mikv_prefill_src* src,
                                   int32_t* demoted_pos, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * One full decode step: mikv_decode_attn followed by the decode mode of
 * mikv_h2o_update_select at the same len (append, attention over both
 * tiers, H2O accumulate, re-select, demote; see those two entry points for
 * the definitions). Results are bit-identical to the two calls; the H2O work
 * runs inside the attention's merge launch when cap16 <= 4096, so the step
 * takes two kernel launches instead of three.
 * q, k_new, v_new, b, o, p16 as in mikv_decode_attn; recent, heavy and
 * demoted_pos (optional) as in mikv_h2o_update_select.
 * ws: mikv_decode_attn_workspace(dims, max_len) bytes.
 * Errors: the union of both entry points' errors.
 */
mikv_status mikv_decode_step(const mikv_dims* dims, const mikv_cache* cache,
                             int32_t len, int32_t recent, int32_t heavy,
                             const uint16_t* q, const uint16_t* k_new,
                             const uint16_t* v_new, const float* b, float* o,
                             float* p16, int32_t* demoted_pos, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * Output-perturbation diagnostic ([gist CriticalKV] theoretical framework:
 * replacing the full cache by a selected part perturbs the attention output
 * by L = ||o - o_hat||_1, bounded through the attention weights and the
 * value states projected by W_O). Per head h, with scale 1/sqrt(d):
 *   o[h]     = softmax over all T tokens of K[h] . q[h], weighting V[h];
 *   o_hat[h] = the same over the kept tokens keep[h][0..n_keep) with the
 *              softmax renormalised over them (an eviction), or, when keep
 *              is NULL, the caller's o_hat[h] (e.g. the output of
 *              mikv_decode_attn on a mixed-precision cache of these tokens);
 *   delta = o - o_hat; L_head[h] = ||delta||_1;
 *   L_proj[h] = ||delta . W_O[h*d .. h*d+d-1][:]||_1 (the head's share of
 *              the layer output, W_O laid out [H*d][hidden]).
 * q [H][d], K, V [H][T][d] fp16, W_O [H*d][hidden] fp16, keep [H][n_keep]
 * int32 (indices in [0, T), each at most once; others are ignored) or NULL,
 * o_hat [H][d] fp32 or NULL: exactly one of keep and o_hat (inputs).
 * o [H][d] fp32 or NULL, delta [H][d] fp32 or NULL, L_head [H], L_proj [H]
 * fp32 (outputs). fp32 accumulation.
 * ws: mikv_perturbation_workspace(H, T, d, hidden) bytes (any contents).
 * Errors: keep and o_hat both or neither given, a required pointer NULL ->
 * MIKV_ERR_NULL; d not 64 or 128 -> MIKV_ERR_UNSUPPORTED; H, T, hidden < 1,
 * n_keep outside [1, T], q/K/V not 16-byte aligned, T*d*2 >= 2^31,
 * hidden*d*2 >= 2^31 - 1024 -> MIKV_ERR_SHAPE; workspace too small ->
 * MIKV_ERR_WORKSPACE.
 */
size_t mikv_perturbation_workspace(int32_t H, int32_t T, int32_t d, int32_t hidden);
mikv_status mikv_output_perturbation(const uint16_t* q, const uint16_t* K,
                                     const uint16_t* V, const uint16_t* W_O,
                                     const int32_t* keep, int32_t n_keep,
                                     const float* o_hat, int32_t H, int32_t T,
                                     int32_t d, int32_t hidden, float* o,
                                     float* delta, float* L_head, float* L_proj,
                                     void* ws, size_t ws_bytes, void* stream);

/*
 * mikv_decode_step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc. Same computation, arguments, outputs and errors as
 * mikv_decode_step, except that the per-split partial results live in a
 * fixed device array of the library (mikv_decode_step_noalloc_limit()
 * bytes, 16 MiB, on every device the library runs on, held until the
 * process ends) instead of a caller workspace. No call allocates or frees
 * memory; the first call on a device looks the array's address up once.
 * Calls on one device share the array: calls that overlap in time on one
 * device (two streams, two host threads) race and give undefined results;
 * calls ordered on one stream are safe. The array needs no initial
 * contents (each call writes what it reads).
 * Errors: as mikv_decode_step; a shape whose partial results exceed the
 * array (mikv_decode_attn_workspace(dims, len) > the limit) ->
 * MIKV_ERR_SCRATCH, nothing enqueued.
 */
size_t mikv_decode_step_noalloc_limit(void);
mikv_status mikv_decode_step_noalloc(const mikv_dims* dims,
                                     const mikv_cache* cache, int32_t len,
                                     int32_t recent, int32_t heavy,
                                     const uint16_t* q, const uint16_t* k_new,
                                     const uint16_t* v_new, const float* b,
                                     float* o, float* p16,
                                     int32_t* demoted_pos, void* stream);

/*
 * CriticalKV two-stage selection per head ([gist CriticalKV] Algorithm 1;
 * theoretical framework: the output perturbation bound depends on the
 * attention weights and the value states projected by W_O).
 *   b1 = floor(alpha * budget) evaluated in double precision (alpha is a
 *   double so that a decimal such as 0.7 is not first rounded to float),
 *   b2 = budget - b1;
 *   S1 = top-b1 of A[h] by (A desc, index asc);
 *   n_i = sum_j | sum_c V[h][i][c] * W_O[h*d + c][j] |  for i not in S1
 *         (fp16 products, fp32 accumulation);
 *   score2[h][i] = A[h][i] * n_i (fp32) for i not in S1, -1 for i in S1;
 *   S2 = top-b2 of the rest by (score2 desc, index asc);
 *   idx[h] = S1 u S2 in ascending order.
 * A [H][T] fp32 (>= 0), V [H][T][d] fp16, W_O [H*d][hidden] fp16 (inputs);
 * idx [H][budget] int32, score2 [H][T] fp32 or NULL (outputs).
 * ws: mikv_criticalkv_workspace(H, T, d, hidden) bytes (any contents): the
 * stage-1 marks and row list, score2 when the caller passes NULL, and a
 * copy of W_O laid out [H][hidden][d] (H*d*hidden*2 bytes).
 * Requires d == 128, hidden % 128 == 0, 1 <= budget <= T, 0 <= alpha <= 1.
 */
size_t mikv_criticalkv_workspace(int32_t H, int32_t T, int32_t d,
                                 int32_t hidden);
mikv_status mikv_criticalkv_select(const float* A, const uint16_t* V,
                                   const uint16_t* W_O, int32_t H, int32_t T,
                                   int32_t d, int32_t hidden, int32_t budget,
                                   double alpha, int32_t* idx, float* score2,
                                   void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MIKV_H */
