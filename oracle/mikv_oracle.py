"""Plain CPU oracle of the MiKV mixed-precision KV-cache path.

TEST INFRASTRUCTURE. This module is the checker: only tests, the smoke check
and the benchmark's CPU-baseline leg may import it. It imports numpy only and
shares no code, table or constant generator with the HIP library.

Sources (cited by page title and section throughout):
  [velog notes]      velog.io post "No Token Left Behind: Reliable KV Cache
                     Compression via Importance-Aware Mixed Precision
                     Quantization", a reader's notes on arXiv 2402.18096.
  [paperlayer]       paperlayer.ai source-linked summary of arXiv 2402.18096v1,
                     "No Token Left Behind ...".
  [gist CriticalKV]  gist.science technical summary of arXiv 2502.03805
                     (CriticalKV).

Precision. Values that the parity tests compare bit for bit (the balancer b,
balanced keys, quantization scale/zero and codes, selections) are discrete
functions of fp16 inputs; they are computed here with one fixed float32
operation sequence (IEEE round-to-nearest-even divide and square root, no
fused multiply-add, no reciprocal multiply, round-half-to-even to integers)
and that sequence is their definition. Everything compared to a tolerance
(scores, softmax, attention output, accumulated scores, projected-value
norms) is computed in float64.

Readings where the pages are silent (each listed with its reason in the
design notes of the repository):
  * quantizer zero point is the group minimum, scale (max-min)/(2^bits-1)
    rounded to fp16, codes are computed from the fp16-stored scale;
  * groups are d/2 contiguous channels for keys and values alike;
  * b = 1 where either channel maximum is zero; b is kept in fp32, q/b too;
  * b is per sequence and per kv head, with the query maximum taken over the
    query heads that share the kv head;
  * every cached key is stored balanced (FP16 tier too); values are not;
  * H2O score = running sum of softmax probabilities over the query heads of
    the group; ties in the important-set ranking go to the lower position;
  * the recent window is the R newest positions, the new token included;
  * tokens in the low-bit tier are never promoted back;
  * CriticalKV: b1 = floor(alpha*budget), b2 = budget-b1, stage-2 score
    A_i * ||V_i W_O,h||_1 with W_O laid out [H*d, hidden];
  * reduced-precision importance tier (imp_bits 8 or 4): the same
    per-token group quantizer; a new token is quantized as it is appended
    and attended to through its codes; a token leaving the tier is
    re-quantized for the retained tier from its codes rebuilt as an fp16
    row (fp32 product, fp32 sum rounded to nearest even, then fp16);
  * per-channel key quantization (key_tile = 64): each retained key channel
    gets its own (scale, zero) over a tile of 64 tokens, by the same
    quantizer rule run along tokens; values stay per token. Demoted pairs
    wait in an fp16 buffer until 64 have gathered, then the buffer becomes
    one tile (keys per channel, values per token); buffered pairs are
    attended to in fp16. At prefill the retained tokens fill tiles in
    ascending position and the last (T-B) mod 64 of them start the buffer.
    The importance tier stays fp16 in this mode.

Parity unpinned (conventions of this repository, not fixed by the pages):
  the bit layout of packed codes, the rounding of the budget split, and the
  synthetic prefill scores acc0 that the decode parity cases start from
  (prefill_scores computes acc0 from q and k; it is pinned by its tests).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "balance", "balance_keys", "quantize_rows", "pack_codes", "unpack_codes",
    "dequantize_rows", "dequantize_rows_f16", "top_by_key", "prefill_build", "decode_attention",
    "h2o_accumulate", "select_drop", "demote", "decode_step",
    "projected_value_l1", "criticalkv_select", "empty_state", "prefill_scores",
    "output_perturbation", "KEY_TILE", "quantize_channels", "dequantize_channels", "retained_counts",
]

F16, F32, F64 = np.float16, np.float32, np.float64


# --------------------------------------------------------------------------
# Channel balancer
# --------------------------------------------------------------------------
def balance(q: np.ndarray, k: np.ndarray):
    """Channel balancer and balanced prompt keys.

    [velog notes] Key contributions 2) "Outlier-aware": during prefill, for
    layer l, head h, channel c, b_lhc is the square root of the ratio of the
    channel's largest |query| to its largest |key| over the prompt tokens 0..t-1
    (balancer equation); keys are multiplied by b before quantization
    (equation for k-hat). [paperlayer] section 3.2: the balancer is computed
    at prefill and applied to keys and queries.

    q: [n, hq, T, d] fp16, k: [n, hkv, T, d] fp16 with hq a multiple of hkv.
    Returns b [n, hkv, d] fp32 and kb [n, hkv, T, d] fp16.
    """
    n, hq, T, d = q.shape
    _, hkv, Tk, dk = k.shape
    assert Tk == T and dk == d and hq % hkv == 0
    rep = hq // hkv
    if T == 0:
        mq = np.zeros((n, hkv, d), F32)
        mk = np.zeros((n, hkv, d), F32)
    else:
        mq = np.abs(q.astype(F32)).reshape(n, hkv, rep, T, d).max(axis=(2, 3))
        mk = np.abs(k.astype(F32)).max(axis=2)
    zero = (mq == 0) | (mk == 0)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (mq / np.where(zero, F32(1), mk)).astype(F32)
    b = np.sqrt(ratio).astype(F32)
    b[zero] = F32(1)
    return b, balance_keys(k, b[:, :, None, :])


def balance_keys(k: np.ndarray, b: np.ndarray) -> np.ndarray:
    """k-hat before quantization: fp16(fp32(k) * b), per channel.

    [velog notes] Key contributions 2), equation for k-hat: the key is
    multiplied by b_lhc. k: [..., d] fp16 whose leading dims broadcast
    against b's [n, hkv, d] once a token axis is inserted by the caller.
    """
    return (k.astype(F32) * b.astype(F32)).astype(F16)


# --------------------------------------------------------------------------
# Per-token asymmetric quantization
# --------------------------------------------------------------------------
def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes [rows, d] into bytes [rows, d*bits/8].

    Little-endian within a byte: code of channel (8/bits)*j + m occupies
    bits [bits*m, bits*m + bits) of byte j.
    """
    per = 8 // bits
    rows, d = codes.shape
    c = codes.astype(np.uint8).reshape(rows, d // per, per)
    out = np.zeros((rows, d // per), np.uint8)
    for m in range(per):
        out |= (c[:, :, m] << (bits * m)).astype(np.uint8)
    return out


def unpack_codes(packed: np.ndarray, d: int, bits: int) -> np.ndarray:
    per = 8 // bits
    rows = packed.shape[0]
    mask = (1 << bits) - 1
    out = np.empty((rows, d // per, per), np.int64)
    for m in range(per):
        out[:, :, m] = (packed >> (bits * m)) & mask
    return out.reshape(rows, d)


def quantize_rows(x: np.ndarray, group: int, bits: int):
    """Per-token asymmetric round-to-nearest quantization with groups.

    [velog notes] Key contributions 1): the retained (evicted) tokens use
    ordinary per-token asymmetric quantization (LLM-QAT style). [velog notes]
    Key contributions 2), additional notes, and [paperlayer] section 3.2: the
    group size is half of the head dimension, to soften RoPE artifacts.

    The same quantizer serves the retained tier (2 or 4 bits) and a
    reduced-precision importance tier (8 or 4 bits, [velog notes] Key
    contributions 3); [paperlayer] section 3.3).

    Per row and group of `group` contiguous channels:
      mn, mx = min, max (exact in fp16)
      s = fp16( (f32(mx) - f32(mn)) / (2^bits - 1) ),  z = mn
      code = clamp(round_half_even((f32(x) - f32(z)) / f32(s)), 0, 2^bits-1)
      (all codes 0 when s == 0; a zero scale or zero point is stored as +0).
    x: [rows, d] fp16. Returns packed codes [rows, d*bits/8] uint8 and
    sz [rows, d/group, 2] fp16 holding (scale, zero) per group.
    """
    assert bits in (2, 4, 8)
    rows, d = x.shape
    assert d % group == 0 and group % (8 // bits) == 0
    qmax = F32((1 << bits) - 1)
    ng = d // group
    xs = x.reshape(rows, ng, group)
    if rows == 0:
        return (np.zeros((0, d * bits // 8), np.uint8), np.zeros((0, ng, 2), F16))
    mn = xs.min(axis=2)
    mx = xs.max(axis=2)
    s32 = ((mx.astype(F32) - mn.astype(F32)) / qmax).astype(F32)
    s16 = s32.astype(F16)
    # signed zeros are stored as +0 so that (scale, zero) bits are unique
    s16[s16 == 0] = F16(0)
    z16 = np.where(mn == 0, F16(0), mn).astype(F16)
    s_safe = np.where(s16 == 0, F32(1), s16.astype(F32)).astype(F32)
    t = ((xs.astype(F32) - z16.astype(F32)[:, :, None]) / s_safe[:, :, None]).astype(F32)
    codes = np.clip(np.rint(t), 0, qmax)
    codes[s16 == 0] = 0
    packed = pack_codes(codes.reshape(rows, d).astype(np.int64), bits)
    sz = np.stack([s16, z16], axis=-1).astype(F16)
    return packed, sz


def dequantize_rows(packed: np.ndarray, sz: np.ndarray, group: int, bits: int) -> np.ndarray:
    """code * scale + zero, in float64. Returns [rows, d]."""
    rows = packed.shape[0]
    d = packed.shape[1] * 8 // bits
    c = unpack_codes(packed, d, bits).astype(F64).reshape(rows, d // group, group)
    s = sz[:, :, 0].astype(F64)[:, :, None]
    z = sz[:, :, 1].astype(F64)[:, :, None]
    return (c * s + z).reshape(rows, d)


def dequantize_rows_f16(packed: np.ndarray, sz: np.ndarray, group: int, bits: int) -> np.ndarray:
    """fp16 rows of codes: fp16(fl32(fl32(code * scale) + zero)).

    A reduced-precision importance tier keeps only codes, so a token that
    leaves it is re-quantized for the retained tier from this fp16 row (the
    fp16 original no longer exists). Reading of this repository: the row is
    rebuilt in fp32 (the product is exact, the sum rounded to nearest even)
    and rounded to fp16, the precision the quantizer takes in."""
    rows = packed.shape[0]
    d = packed.shape[1] * 8 // bits
    c = unpack_codes(packed, d, bits).astype(F32).reshape(rows, d // group, group)
    s = sz[:, :, 0].astype(F32)[:, :, None]
    z = sz[:, :, 1].astype(F32)[:, :, None]
    return ((c * s).astype(F32) + z).astype(F32).astype(F16).reshape(rows, d)


# --------------------------------------------------------------------------
# Per-channel key quantization over token tiles
# --------------------------------------------------------------------------
KEY_TILE = 64


def quantize_channels(x: np.ndarray, bits: int):
    """Per-channel asymmetric quantization of a tile of keys.

    [velog notes] Alternative approach (per-channel quantization) and its
    appendix C summary; [paperlayer] appendix C: keys may instead be
    quantized per channel, which isolates outlier channels, with groups of
    64 along the tokens. The rule is the per-token quantizer's (quantize_rows)
    applied to each channel's column of the tile: every channel c gets
    s_c = fp16((max - min) / (2^bits - 1)) and z_c = min over the t tokens.

    x: [t, d] fp16 (one tile). Returns packed codes [t, d*bits/8] in the
    per-token byte layout (token-major, channels packed within a row) and
    sz [d, 2] fp16 holding (scale, zero) per channel.
    """
    t, d = x.shape
    packed_c, sz = quantize_rows(np.ascontiguousarray(x.T), t, bits)   # rows = channels
    codes = unpack_codes(packed_c, t, bits).T                            # [t, d]
    return pack_codes(np.ascontiguousarray(codes), bits), sz[:, 0, :].copy()


def dequantize_channels(packed: np.ndarray, sz: np.ndarray, bits: int) -> np.ndarray:
    """code * scale_c + zero_c of a tile, float64 [t, d]."""
    d = sz.shape[0]
    c = unpack_codes(packed, d, bits).astype(F64)
    return c * sz[:, 0].astype(F64)[None, :] + sz[:, 1].astype(F64)[None, :]


def retained_counts(st, D):
    """(tokens in full tiles, tokens in the buffer) of a per-channel cache
    whose retained tier has taken D tokens; (D, 0) for per-token keys."""
    kt = st.get("key_tile", 0)
    if not kt:
        return D, 0
    return kt * (D // kt), D % kt


def _put_tile(st, i, g, j, krows, vrows, pos):
    """Quantize a full tile of retained pairs into tile j: keys per channel,
    values per token (group d/2 like every value row)."""
    kt, bits, group = st["key_tile"], st["bits"], st["group"]
    sl = slice(j * kt, (j + 1) * kt)
    st["kq"][i, g, sl], st["kcsz"][i, g, j] = quantize_channels(krows, bits)
    st["vq"][i, g, sl], st["vsz"][i, g, sl] = quantize_rows(vrows, group, bits)
    st["posq"][i, g, sl] = pos


def _retained_kv(st, i, g, D):
    """Keys and values (float64) of the retained tokens of unit (i, g), in
    the order they left the importance tier: the low-bit slots, then (per-
    channel keys) the buffered pairs."""
    group, bits = st["group"], st["bits"]
    nq, nb = retained_counts(st, D)
    if not st.get("key_tile", 0):
        return (dequantize_rows(st["kq"][i, g, :nq], st["ksz"][i, g, :nq], group, bits),
                dequantize_rows(st["vq"][i, g, :nq], st["vsz"][i, g, :nq], group, bits))
    kt = st["key_tile"]
    K = [dequantize_channels(st["kq"][i, g, j * kt:(j + 1) * kt], st["kcsz"][i, g, j], bits)
         for j in range(nq // kt)]
    K.append(st["kbuf"][i, g, :nb].astype(F64))
    V = dequantize_rows(st["vq"][i, g, :nq], st["vsz"][i, g, :nq], group, bits)
    return np.concatenate(K), np.concatenate([V, st["vbuf"][i, g, :nb].astype(F64)])


# --------------------------------------------------------------------------
# Importance ranking (H2O heavy hitters)
# --------------------------------------------------------------------------
def top_by_key(score: np.ndarray, pos: np.ndarray, m: int) -> np.ndarray:
    """Indices of the m best entries by (score descending, position ascending).

    The importance-based eviction the MiKV notes use is H2O ([velog notes]
    Key contributions 1)); heavy hitters are the tokens with the largest
    accumulated attention ([paperlayer] section 5, KV cache eviction). Equal
    scores are ranked by lower token position.
    """
    order = np.lexsort((pos, -score.astype(F64)))
    return order[:m]


def empty_state(batch, hkv, d, cap16, capq, group, bits, imp_bits=16, key_tile=0):
    """Zeroed cache in the layout of the C interface (see include/mikv.h).

    imp_bits = 16: the importance tier holds fp16 rows (k16, v16). imp_bits
    in (8, 4): it holds codes and (scale, zero) like the retained tier
    (kimp, vimp, kimpsz, vimpsz), the reduced-precision importance cache of
    [velog notes] Key contributions 3) and [paperlayer] section 3.3.

    key_tile = 64: retained keys are quantized per channel over tiles of 64
    tokens (kcsz [n, hkv, capq/64, d, 2] in place of ksz), with an fp16
    buffer (kbuf, vbuf [n, hkv, 64, d], posbuf) for pairs that wait for a
    tile to fill ([velog notes] appendix C summary: a temporary buffer,
    kept apart from the important pairs)."""
    cb = d * bits // 8
    st = dict(
        pos16=np.full((batch, hkv, cap16), -1, np.int32),
        acc16=np.zeros((batch, hkv, cap16), F32),
        free16=np.zeros((batch, hkv), np.int32),
        kq=np.zeros((batch, hkv, capq, cb), np.uint8), vq=np.zeros((batch, hkv, capq, cb), np.uint8),
        vsz=np.zeros((batch, hkv, capq, d // group, 2), F16),
        posq=np.full((batch, hkv, capq), -1, np.int32),
        group=group, bits=bits, imp_bits=imp_bits, key_tile=key_tile,
    )
    if key_tile:
        assert key_tile == KEY_TILE and capq % key_tile == 0 and imp_bits == 16
        st["kcsz"] = np.zeros((batch, hkv, capq // key_tile, d, 2), F16)
        st["kbuf"] = np.zeros((batch, hkv, key_tile, d), F16)
        st["vbuf"] = np.zeros((batch, hkv, key_tile, d), F16)
        st["posbuf"] = np.full((batch, hkv, key_tile), -1, np.int32)
    else:
        st["ksz"] = np.zeros((batch, hkv, capq, d // group, 2), F16)
    if imp_bits == 16:
        st["k16"] = np.zeros((batch, hkv, cap16, d), F16)
        st["v16"] = np.zeros((batch, hkv, cap16, d), F16)
    else:
        assert imp_bits in (4, 8)
        ci = d * imp_bits // 8
        st["kimp"] = np.zeros((batch, hkv, cap16, ci), np.uint8)
        st["vimp"] = np.zeros((batch, hkv, cap16, ci), np.uint8)
        st["kimpsz"] = np.zeros((batch, hkv, cap16, d // group, 2), F16)
        st["vimpsz"] = np.zeros((batch, hkv, cap16, d // group, 2), F16)
    return st


def _shape(st):
    n, hkv, cap16 = st["pos16"].shape
    return n, hkv, cap16, st["kq"].shape[-1] * 8 // st["bits"]


def _imp_bits(st):
    return st.get("imp_bits", 16)


def _imp_kv(st, i, g):
    """Keys and values of the importance tier of unit (i, g), float64."""
    ib = _imp_bits(st)
    if ib == 16:
        return st["k16"][i, g].astype(F64), st["v16"][i, g].astype(F64)
    grp = st["group"]
    return (dequantize_rows(st["kimp"][i, g], st["kimpsz"][i, g], grp, ib),
            dequantize_rows(st["vimp"][i, g], st["vimpsz"][i, g], grp, ib))


def _imp_put(st, i, g, slots, krows, vrows):
    """Store fp16 rows [m, d] into importance-tier slots (quantized when the
    tier is reduced-precision)."""
    ib = _imp_bits(st)
    if ib == 16:
        st["k16"][i, g, slots] = krows
        st["v16"][i, g, slots] = vrows
        return
    grp = st["group"]
    ck, sk = quantize_rows(krows, grp, ib)
    cv, sv = quantize_rows(vrows, grp, ib)
    st["kimp"][i, g, slots], st["kimpsz"][i, g, slots] = ck, sk
    st["vimp"][i, g, slots], st["vimpsz"][i, g, slots] = cv, sv


def _imp_rows16(st, i, g, s):
    """fp16 key and value rows of importance slot s: the stored rows, or the
    codes rebuilt as fp16 (dequantize_rows_f16) for a reduced-precision
    tier."""
    ib = _imp_bits(st)
    if ib == 16:
        return st["k16"][i, g, s:s + 1], st["v16"][i, g, s:s + 1]
    grp = st["group"]
    return (dequantize_rows_f16(st["kimp"][i, g, s:s + 1], st["kimpsz"][i, g, s:s + 1], grp, ib),
            dequantize_rows_f16(st["vimp"][i, g, s:s + 1], st["vimpsz"][i, g, s:s + 1], grp, ib))


def prefill_build(kb, v, acc0, B, R, group, bits, capq, imp_bits=16, key_tile=0):
    """Initial two-tier cache after the prompt.

    [velog notes] one-line summary and Key contributions 1): tokens an
    importance-based eviction would drop are kept at low precision; important
    tokens stay at high precision. Important set = the R newest positions
    plus the top-(B-R) older positions by accumulated attention (H2O heavy
    hitters and local tokens, [paperlayer] section 5). The FP16 tier holds
    the important set in ascending position (slots 0..B-1, slot B free); the
    low-bit tier holds the others in ascending position. Grouping pairs by
    precision is allowed because attention is permutation invariant
    ([velog notes] section 3.4).

    kb, v: [n, hkv, T, d] fp16 (balanced keys, values); acc0 [n, hkv, T] fp32.
    imp_bits < 16: the important rows are stored as imp_bits codes.
    key_tile = 64: the retained tokens fill per-channel key tiles in
    ascending position; the last (T-B) mod 64 of them go to the buffer.
    """
    n, hkv, T, d = kb.shape
    H = B - R
    assert 0 <= R <= B <= T and T - B <= capq
    st = empty_state(n, hkv, d, B + 1, capq, group, bits, imp_bits, key_tile)
    pos_all = np.arange(T, dtype=np.int64)
    for i in range(n):
        for g in range(hkv):
            cand = pos_all[:T - R]
            heavy = cand[top_by_key(acc0[i, g, :T - R], cand, H)]
            keep = np.zeros(T, bool)
            keep[heavy] = True
            keep[T - R:] = True
            kp = pos_all[keep]
            rp = pos_all[~keep]
            _imp_put(st, i, g, slice(0, B), kb[i, g, kp], v[i, g, kp])
            st["pos16"][i, g, :B] = kp
            st["acc16"][i, g, :B] = acc0[i, g, kp]
            st["free16"][i, g] = B
            if key_tile:
                nq, nb = retained_counts(st, len(rp))
                for j in range(nq // key_tile):
                    tp = rp[j * key_tile:(j + 1) * key_tile]
                    _put_tile(st, i, g, j, kb[i, g, tp], v[i, g, tp], tp)
                st["kbuf"][i, g, :nb] = kb[i, g, rp[nq:]]
                st["vbuf"][i, g, :nb] = v[i, g, rp[nq:]]
                st["posbuf"][i, g, :nb] = rp[nq:]
                continue
            ck, sk = quantize_rows(kb[i, g, rp], group, bits)
            cv, sv = quantize_rows(v[i, g, rp], group, bits)
            m = len(rp)
            st["kq"][i, g, :m], st["ksz"][i, g, :m] = ck, sk
            st["vq"][i, g, :m], st["vsz"][i, g, :m] = cv, sv
            st["posq"][i, g, :m] = rp
    return st


# --------------------------------------------------------------------------
# Decode step
# --------------------------------------------------------------------------
def decode_attention(state, N, q, k_new, v_new, b):
    """Append the new token, then attention over both precision tiers.

    [velog notes] section 3.4 and [paperlayer] section 3.4: decode attention
    is a batch matrix-vector product; keys and values are stored at reduced
    precision while the query and the attention map stay floating point.
    [velog notes] Key contributions 2): the query is divided by b (q-hat) and
    the key was multiplied by b, so q-hat . k-hat reproduces q . k. With a
    reduced-precision importance tier the new token is stored as codes and
    attended to through them, like every other importance-tier token.
    Scores use scale 1/sqrt(d); the new token attends to every cached token
    and to itself. With per-channel keys the retained tokens are the full
    tiles (keys code * scale_c + zero_c) and the buffered fp16 pairs.

    state: cache dict (see empty_state) before the step; the retained tier
    holds N - cap16 tokens and slot free16 of the FP16 tier is free.
    q [n, hq, d], k_new/v_new [n, hkv, d] fp16; b [n, hkv, d] fp32.
    Returns (o [n,hq,d] f64, p16 [n,hkv,cap16] f64 summed over the group's
    query heads, pq [n,hkv,N-cap16] f64 likewise for the retained tokens in
    the order they were demoted, appended state).
    """
    st = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in state.items()}
    group, bits = st["group"], st["bits"]
    n, hkv, cap16, d = _shape(st)
    hq = q.shape[1]
    rep = hq // hkv
    nq = N - cap16
    assert nq >= 0
    o = np.zeros((n, hq, d), F64)
    p16 = np.zeros((n, hkv, cap16), F64)
    pq = np.zeros((n, hkv, nq), F64)
    for i in range(n):
        for g in range(hkv):
            s = int(st["free16"][i, g])
            _imp_put(st, i, g, slice(s, s + 1), balance_keys(k_new[i, g], b[i, g])[None],
                     v_new[i, g][None])
            st["pos16"][i, g, s] = N - 1
            st["acc16"][i, g, s] = 0.0
            Ki, Vi = _imp_kv(st, i, g)
            Kr, Vr = _retained_kv(st, i, g, nq)
            K = np.concatenate([Ki, Kr])
            V = np.concatenate([Vi, Vr])
            for r in range(rep):
                h = g * rep + r
                qh = q[i, h].astype(F64) / b[i, g].astype(F64)
                sc = (K @ qh) / np.sqrt(F64(d))
                e = np.exp(sc - sc.max())
                p = e / e.sum()
                o[i, h] = p @ V
                p16[i, g] += p[:cap16]
                pq[i, g] += p[cap16:]
    return o, p16, pq, st


def prefill_scores(q, k):
    """Heavy-hitter scores of the prompt tokens (acc0), float64.

    [paperlayer] section 5: a token's importance is the attention it has
    accumulated. Over the prompt this is taken as: for every query head h of
    the group and every query position i, the causal softmax of
    q_i . k_t / sqrt(d) over t <= i; acc0[t] sums those weights over the
    group's heads and over the queries i >= t. The plain reading of
    "accumulated attention" at prefill (the pages give no separate formula):
    the same sum the decode steps keep adding to, started from the prompt.

    q [n, hq, T, d], k [n, hkv, T, d] (fp16 values) -> acc0 [n, hkv, T].
    """
    n, hq, T, d = q.shape
    hkv = k.shape[1]
    rep = hq // hkv
    acc = np.zeros((n, hkv, T), F64)
    later = np.triu(np.ones((T, T), bool), 1)   # key t > query i
    for i in range(n):
        for h in range(hq):
            g = h // rep
            s = (q[i, h].astype(F64) @ k[i, g].astype(F64).T) / np.sqrt(F64(d))
            s[later] = -np.inf
            e = np.exp(s - s.max(axis=1, keepdims=True))
            acc[i, g] += (e / e.sum(axis=1, keepdims=True)).sum(axis=0)
    return acc


def h2o_accumulate(acc16, p16):
    """acc += probability mass of this step (float64). [paperlayer] section 5:
    heavy hitters are ranked by accumulated attention."""
    return acc16.astype(F64) + p16


def select_drop(acc, pos16, N, R, H):
    """Slot to demote per (n, g) after one decode step.

    The FP16 tier holds the R newest positions (the window, new token
    included) and H+1 older candidates. Re-selecting the top-H candidates by
    (acc desc, position asc) leaves exactly one candidate out; that one is
    demoted. Returns drop [n, hkv] int64 (slot index).
    """
    n, hkv, cap16 = pos16.shape
    drop = np.empty((n, hkv), np.int64)
    for i in range(n):
        for g in range(hkv):
            cand = np.nonzero(pos16[i, g] < N - R)[0]
            assert len(cand) == H + 1, (len(cand), H)
            keep = cand[top_by_key(acc[i, g, cand], pos16[i, g, cand], H)]
            rest = np.setdiff1d(cand, keep)
            assert len(rest) == 1
            drop[i, g] = rest[0]
    return drop


def demote(state, N, drop):
    """Quantize each dropped importance-tier token into low-bit slot N - cap16.

    [velog notes] Key contributions 1): tokens leaving the important set are
    kept as low-bit codes instead of being discarded. From a reduced-precision
    importance tier the row re-quantized is its codes rebuilt in fp16
    (dequantize_rows_f16). With per-channel keys the pair goes to buffer row
    (N - cap16) mod 64 instead; the pair that fills the buffer turns it into
    tile (N - cap16) // 64 ([velog notes] appendix C summary: pairs wait in
    a temporary buffer until enough have gathered, then are quantized).
    """
    st = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in state.items()}
    group, bits = st["group"], st["bits"]
    n, hkv, cap16, d = _shape(st)
    slot = N - cap16
    kt = st.get("key_tile", 0)
    for i in range(n):
        for g in range(hkv):
            s = int(drop[i, g])
            krow, vrow = _imp_rows16(st, i, g, s)
            if kt:
                r = slot % kt
                st["kbuf"][i, g, r], st["vbuf"][i, g, r] = krow[0], vrow[0]
                st["posbuf"][i, g, r] = st["pos16"][i, g, s]
                if r == kt - 1:
                    _put_tile(st, i, g, slot // kt, st["kbuf"][i, g], st["vbuf"][i, g], st["posbuf"][i, g])
                st["free16"][i, g] = s
                continue
            ck, sk = quantize_rows(krow, group, bits)
            cv, sv = quantize_rows(vrow, group, bits)
            st["kq"][i, g, slot], st["ksz"][i, g, slot] = ck[0], sk[0]
            st["vq"][i, g, slot], st["vsz"][i, g, slot] = cv[0], sv[0]
            st["posq"][i, g, slot] = st["pos16"][i, g, s]
            st["free16"][i, g] = s
    return st


def decode_step(state, N, q, k_new, v_new, b, R, H):
    """One full decode step: append, attention, accumulate, re-select, demote.
    Returns (o, p16, new_state, drop)."""
    o, p16, _, st = decode_attention(state, N, q, k_new, v_new, b)
    acc = h2o_accumulate(st["acc16"], p16)
    st["acc16"] = acc.astype(F32)
    drop = select_drop(acc, st["pos16"], N, R, H)
    return o, p16, demote(st, N, drop), drop


# --------------------------------------------------------------------------
# CriticalKV two-stage selection
# --------------------------------------------------------------------------
def projected_value_l1(V, W_O, rows=None, chunk=2048):
    """n_i = || V_h[i,:] @ W_O[h*d:(h+1)*d, :] ||_1 per head (float64).

    [gist CriticalKV] theoretical framework: the output-perturbation bound
    depends on the attention weights and on the value states projected by the
    output matrix W_O. V: [H, T, d] fp16; W_O: [H*d, hidden] fp16.
    Returns [H, T] float64 (rows outside `rows[h]`, if given, are left 0).
    """
    H, T, d = V.shape
    out = np.zeros((H, T), F64)
    for h in range(H):
        Wh = W_O[h * d:(h + 1) * d].astype(F64)
        idx = np.arange(T) if rows is None else np.asarray(rows[h])
        for c0 in range(0, len(idx), chunk):
            sl = idx[c0:c0 + chunk]
            out[h, sl] = np.abs(V[h, sl].astype(F64) @ Wh).sum(axis=1)
    return out


def criticalkv_select(A, V, W_O, budget, alpha, norms=None, score2=None):
    """CriticalKV perturbation-constrained two-stage selection per head.

    [gist CriticalKV] Algorithm 1: stage 1 spends b' = alpha * b of the
    budget on the entries with the largest attention weight A_i; stage 2
    spends the remaining b'' on the entries maximising A_i times the L1 norm
    of the projected value state (V_i W_O). Ties go to the lower index.

    A [H, T] fp32, V [H, T, d] fp16, W_O [H*d, hidden] fp16.
    Returns idx [H, budget] (ascending), score2 [H, T] float64 (A_i * n_i for
    entries outside stage 1, -1 for stage-1 entries) and s1 mask [H, T].
    `norms` may pass precomputed n [H, T] (rows outside stage 1 are used);
    `score2` may pass a stage-2 score array to rank instead (its stage-1
    entries are ignored), which is how a device result is re-ranked.
    """
    H, T = A.shape
    assert 1 <= budget <= T and 0.0 <= alpha <= 1.0
    b1 = int(np.floor(F64(alpha) * budget))
    b2 = budget - b1
    pos = np.arange(T)
    s1 = np.zeros((H, T), bool)
    for h in range(H):
        s1[h, top_by_key(A[h], pos, b1)] = True
    if score2 is None:
        if norms is None:
            norms = projected_value_l1(V, W_O, rows=[pos[~s1[h]] for h in range(H)])
        score2 = A.astype(F64) * norms
    score2 = np.where(s1, -1.0, np.asarray(score2, F64))
    idx = np.empty((H, budget), np.int64)
    for h in range(H):
        rest = pos[~s1[h]]
        sel2 = rest[top_by_key(score2[h, rest], rest, b2)]
        idx[h] = np.sort(np.concatenate([pos[s1[h]], sel2]))
    return idx, score2, s1


# --------------------------------------------------------------------------
# Output-perturbation diagnostic
# --------------------------------------------------------------------------
def output_perturbation(q, K, V, W_O, keep=None, o_hat=None):
    """L = ||o - o_hat||_1 per head, in head space and after W_O,h (float64).

    [gist CriticalKV] theoretical framework: the perturbation of replacing
    the full cache by a selected part is the L1 distance between the
    attention outputs, and its bound involves the attention weights and the
    value states projected by W_O. Reading of this repository: o is the
    head's softmax attention over all T tokens (scale 1/sqrt(d)); o_hat is
    either the attention over the kept tokens `keep[h]` with the softmax
    renormalized over them (an eviction: H2O, CriticalKV) or a given output
    (a compressed cache such as MiKV's mixed precision); the projected
    perturbation is ||(o - o_hat) W_O,h||_1 with W_O,h = rows h*d..h*d+d-1
    of W_O [H*d, hidden].

    q [H, d], K, V [H, T, d] (fp16 values), W_O [H*d, hidden]; keep: list of
    index arrays or None; o_hat [H, d] or None. Returns (o [H, d],
    o_hat [H, d], L_head [H], L_proj [H]).
    """
    H, T, d = K.shape
    assert (keep is None) != (o_hat is None)
    o = np.zeros((H, d), F64)
    oh = np.zeros((H, d), F64)
    L_head = np.zeros(H, F64)
    L_proj = np.zeros(H, F64)
    for h in range(H):
        s = (K[h].astype(F64) @ q[h].astype(F64)) / np.sqrt(F64(d))
        e = np.exp(s - s.max())
        o[h] = (e / e.sum()) @ V[h].astype(F64)
        if keep is not None:
            sel = np.asarray(keep[h])
            es = np.exp(s[sel] - s[sel].max())
            oh[h] = (es / es.sum()) @ V[h, sel].astype(F64)
        else:
            oh[h] = np.asarray(o_hat[h], F64)
        delta = o[h] - oh[h]
        L_head[h] = np.abs(delta).sum()
        L_proj[h] = np.abs(delta @ W_O[h * d:(h + 1) * d].astype(F64)).sum()
    return o, oh, L_head, L_proj
