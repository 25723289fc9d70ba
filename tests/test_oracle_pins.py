"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values
derived by hand (tests/golden), closed forms on planted inputs, invariants
(balancer identity, permutation invariance, probability conservation),
library routines for special cases (scaled-dot-product attention in float64)
and brute force over all subsets on tiny inputs.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_decode_amd import synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F16, F32, F64 = np.float16, np.float32, np.float64


# ---------------------------------------------------------------- balancer
def _small_qk(rng, n, hq, hkv, T, d):
    q = (rng.uniform(-0.5, 0.5, (n, hq, T, d))).astype(F16)
    k = (rng.uniform(-0.5, 0.5, (n, hkv, T, d))).astype(F16)
    return q, k


def test_balancer_planted_maxima_closed_form():
    """b = sqrt(max|q| / max|k|): plant the channel maxima so b is known exactly.

    The q maximum is planted in a random query head of the group (often the
    last one) and a random token, so a wrong head-to-group mapping or a
    missing token range changes b."""
    rng = np.random.default_rng(7)
    n, hq, hkv, T, d = 2, 8, 2, 6, 8
    rep = hq // hkv
    q, k = _small_qk(rng, n, hq, hkv, T, d)
    ratios = [(4.0, 1.0, 2.0), (1.0, 4.0, 0.5), (2.0, 2.0, 1.0), (16.0, 1.0, 4.0),
              (9.0, 1.0, 3.0), (1.0, 16.0, 0.25), (8.0, 2.0, 2.0), (3.0, 12.0, 0.5)]
    expect = np.empty((n, hkv, d), F32)
    for i in range(n):
        for g in range(hkv):
            for c in range(d):
                mq, mk, bb = ratios[(i * 3 + g * 5 + c) % len(ratios)]
                h = g * rep + (rep - 1 if c % 2 == 0 else int(rng.integers(rep)))
                t = int(rng.integers(T))
                q[i, h, t, c] = F16(-mq if c % 3 == 0 else mq)
                k[i, g, int(rng.integers(T)), c] = F16(mk if c % 2 else -mk)
                expect[i, g, c] = bb
    b, kb = O.balance(q, k)
    assert b.dtype == F32 and np.array_equal(b, expect)
    # keys are multiplied (not divided) by b; these products are exact in fp16
    exact = np.isin(expect, [0.25, 0.5, 1.0, 2.0, 4.0])
    prod = (k.astype(F64) * expect[:, :, None, :].astype(F64))
    m = np.broadcast_to(exact[:, :, None, :], prod.shape)
    assert np.array_equal(kb.astype(F64)[m], prod[m])


def test_balancer_zero_guard_and_empty_prompt():
    rng = np.random.default_rng(1)
    q, k = _small_qk(rng, 1, 2, 1, 5, 4)
    k[0, 0, :, 1] = 0          # key channel identically zero
    q[0, :, :, 2] = 0          # query channel identically zero
    b, _ = O.balance(q, k)
    assert b[0, 0, 1] == 1.0 and b[0, 0, 2] == 1.0
    b0, kb0 = O.balance(q[:, :, :0], k[:, :, :0])
    assert np.all(b0 == 1.0) and kb0.shape == (1, 1, 0, 4)


def test_balancer_q_equals_k_gives_one():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 3, 17, 8)).astype(F16)
    b, kb = O.balance(x, x.copy())
    assert np.all(b == 1.0) and np.array_equal(kb, x)


def test_balancer_equalises_channel_ranges():
    """After balancing, the largest |k*b| and the largest |q/b| of a channel
    both equal sqrt(max|q| * max|k|) (the geometric mean): the purpose stated
    for b on the velog notes page (K side range shrinks, Q absorbs it)."""
    cfg = S.CONFIGS["tiny"].scaled(hq=4, hkv=2, d=64, T=64)
    q, k, _, _ = S.prefill_tensors(cfg, 11)
    b, _ = O.balance(q, k)
    mq = np.abs(q.astype(F64)).reshape(1, 2, 2, 64, 64).max(axis=(2, 3))
    mk = np.abs(k.astype(F64)).max(axis=2)
    gm = np.sqrt(mq * mk)
    np.testing.assert_allclose(mk * b, gm, rtol=1e-6)
    np.testing.assert_allclose(mq / b, gm, rtol=1e-6)


def test_balancer_identity_before_quantization():
    """(q / b) . (k * b) == q . k in float64 (velog notes, k-hat / q-hat equations)."""
    cfg = S.CONFIGS["tiny"].scaled(hq=2, hkv=1, T=48)
    q, k, _, _ = S.prefill_tensors(cfg, 3)
    b, _ = O.balance(q, k)
    bb = b.astype(F64)[0, 0]
    qq = q.astype(F64)[0, 0]
    kk = k.astype(F64)[0, 0]
    lhs = (qq / bb) @ (kk * bb).T
    rhs = qq @ kk.T
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))
    assert not np.all(b == 1.0)


# ---------------------------------------------------------------- quantizer
def _golden_cases():
    with open(os.path.join(GOLDEN, "quantizer_hand_vectors.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_quantizer_hand_vectors(case):
    x = np.array(case["x"], F16)[None, :]
    packed, sz = O.quantize_rows(x, case["group"], case["bits"])
    assert sz[0, :, 0].astype(F64).tolist() == case["scale"]
    assert sz[0, :, 1].astype(F64).tolist() == case["zero"]
    assert packed[0].tobytes().hex() == case["packed_hex"].replace(" ", "")
    d = x.shape[1]
    assert O.unpack_codes(packed, d, case["bits"])[0].tolist() == case["codes"]


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("group", [32, 64])
def test_quantizer_roundtrip_bound(bits, group):
    """|x - dequant(quant(x))| <= scale/2 for every element (round to nearest
    with the stored fp16 scale), codes in [0, 2^bits - 1], min -> code 0."""
    rng = np.random.default_rng(5)
    rows, d = 2000, 64
    x = rng.standard_normal((rows, d)).astype(F32)
    x[:, [3, 35]] *= 20
    x[::7] *= 1e-3
    x[::11] *= 500
    x = x.astype(F16)
    x[5, :] = F16(0.75)                      # constant row
    packed, sz = O.quantize_rows(x, group, bits)
    xr = O.dequantize_rows(packed, sz, group, bits)
    s = np.repeat(sz[:, :, 0].astype(F64), group, axis=1)
    err = np.abs(xr - x.astype(F64))
    slack = 1e-6 * (np.abs(x.astype(F64)) + s)
    # the stored scale is the fp16 rounding of range/qmax: when it rounds
    # down, the group maximum lies up to qmax * (range/qmax - s) above the
    # top code and is clamped there (noticeable at 8 bits and subnormal scales)
    qmax = (1 << bits) - 1
    xs64 = x.astype(F64).reshape(rows, d // group, group)
    s_true = (xs64.max(axis=2) - xs64.min(axis=2)) / qmax
    over = np.repeat(np.maximum(0.0, s_true - sz[:, :, 0].astype(F64)) * qmax, group, axis=1)
    assert np.all(err <= 0.5 * s + over + slack)
    codes = O.unpack_codes(packed, d, bits)
    assert codes.min() >= 0 and codes.max() <= (1 << bits) - 1
    xs = x.reshape(rows, d // group, group)
    cs = codes.reshape(rows, d // group, group)
    am = xs.argmin(axis=2)
    assert np.all(np.take_along_axis(cs, am[:, :, None], 2) == 0)
    assert np.array_equal(xr[5], np.full(d, 0.75))


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_pack_unpack_roundtrip(bits):
    rng = np.random.default_rng(9)
    c = rng.integers(0, 1 << bits, (13, 128))
    assert np.array_equal(O.unpack_codes(O.pack_codes(c, bits), 128, bits), c)


def test_quantizer_empty():
    p, sz = O.quantize_rows(np.zeros((0, 64), F16), 32, 4)
    assert p.shape == (0, 32) and sz.shape == (0, 2, 2)


# ---------------------------------------------------------------- selection
def _dominates(a1, p1, a2, p2):
    return a1 > a2 or (a1 == a2 and p1 < p2)


def _brute_top(score, pos, m):
    """Unique subset of size m whose members all outrank every non-member."""
    idx = range(len(score))
    found = []
    for S_ in itertools.combinations(idx, m):
        rest = [j for j in idx if j not in S_]
        if all(_dominates(score[i], pos[i], score[j], pos[j]) for i in S_ for j in rest):
            found.append(sorted(S_))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(6))
def test_top_by_key_brute_force(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 11))
    score = rng.integers(0, 4, T).astype(F32) * F32(0.25)    # many ties
    pos = rng.permutation(50)[:T]
    for m in range(T + 1):
        got = sorted(O.top_by_key(score, pos, m).tolist())
        assert got == _brute_top(score, pos, m)


def test_prefill_build_brute_force_tiny():
    rng = np.random.default_rng(4)
    T, d, B, R = 11, 8, 6, 2
    kb = rng.standard_normal((1, 1, T, d)).astype(F16)
    v = rng.standard_normal((1, 1, T, d)).astype(F16)
    acc0 = (rng.integers(0, 3, (1, 1, T)) * 0.5).astype(F32)
    st = O.prefill_build(kb, v, acc0, B, R, 4, 4, T)
    heavy = _brute_top(acc0[0, 0, :T - R], np.arange(T - R), B - R)
    keep = sorted(heavy + list(range(T - R, T)))
    assert st["pos16"][0, 0, :B].tolist() == keep and st["free16"][0, 0] == B
    rest = [p for p in range(T) if p not in keep]
    assert st["posq"][0, 0, :T - B].tolist() == rest
    assert np.array_equal(st["k16"][0, 0, :B], kb[0, 0, keep])
    assert np.array_equal(st["acc16"][0, 0, :B], acc0[0, 0, keep])


def test_decode_drop_is_minimum_key():
    """Re-selecting top-H of H+1 candidates == dropping the candidate with the
    smallest accumulated score (latest position among equal scores)."""
    rng = np.random.default_rng(12)
    for _ in range(50):
        cap16, R, N = 9, 3, 40
        H = cap16 - 1 - R
        pos = rng.permutation(N - R)[:H + 1].tolist() + list(range(N - R, N))
        pos = np.array(pos, np.int32)[rng.permutation(cap16)][None, None]
        acc = rng.integers(0, 3, (1, 1, cap16)).astype(F64)
        drop = O.select_drop(acc, pos, N, R, H)[0, 0]
        cand = [s for s in range(cap16) if pos[0, 0, s] < N - R]
        worst = min(cand, key=lambda s: (acc[0, 0, s], -pos[0, 0, s]))
        assert drop == worst


# ---------------------------------------------------------------- attention
def _sdpa(q, K, V):
    """Textbook softmax attention in float64 via the library routine."""
    qt = torch.from_numpy(np.ascontiguousarray(q, F64))[None, None, None]
    Kt = torch.from_numpy(np.ascontiguousarray(K, F64))[None, None]
    Vt = torch.from_numpy(np.ascontiguousarray(V, F64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt)[0, 0, 0].numpy()


def _build(cfg, seed, balanced=True):
    q, k, v, acc0 = S.prefill_tensors(cfg, seed)
    if balanced:
        b, kb = O.balance(q, k)
    else:
        b = np.ones((cfg.batch, cfg.hkv, cfg.d), F32)
        kb = k
    st = O.prefill_build(kb, v, acc0, cfg.B, cfg.recent, cfg.G, cfg.bits, cfg.capq())
    return st, b, (q, k, v)


def test_all_fp16_attention_equals_full_attention():
    """Importance share 100% (empty low-bit tier), b = 1: the mixed attention
    is plain softmax attention over prompt + new token."""
    cfg = S.CONFIGS["tiny"].scaled(hq=2, hkv=1, T=40, pct=100, recent=8, factor=3.0)
    st, b, (_, k, v) = _build(cfg, 21, balanced=False)
    qd, kd, vd = S.decode_tensors(cfg, 21, 0)
    N = cfg.T + 1
    o, p16, pq, _ = O.decode_attention(st, N, qd, kd, vd, b)
    assert pq.shape[-1] == 0
    K = np.concatenate([k[0, 0], kd[0, :1]]).astype(F64)
    V = np.concatenate([v[0, 0], vd[0, :1]]).astype(F64)
    for h in range(2):
        ref = _sdpa(qd[0, h].astype(F64), K, V)
        assert np.max(np.abs(o[0, h] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_balanced_attention_matches_unbalanced_within_fp16_key_rounding():
    cfg = S.CONFIGS["tiny"].scaled(hq=2, hkv=1, T=40, pct=100, recent=8, factor=3.0)
    st, b, (_, k, v) = _build(cfg, 22, balanced=True)
    assert not np.all(b == 1)
    qd, kd, vd = S.decode_tensors(cfg, 22, 0)
    o, _, _, _ = O.decode_attention(st, cfg.T + 1, qd, kd, vd, b)
    K = np.concatenate([k[0, 0], kd[0, :1]]).astype(F64)
    V = np.concatenate([v[0, 0], vd[0, :1]]).astype(F64)
    for h in range(2):
        ref = _sdpa(qd[0, h].astype(F64), K, V)
        assert np.max(np.abs(o[0, h] - ref)) <= 1e-2 * np.max(np.abs(ref))


@pytest.mark.parametrize("bits", [4, 2])
def test_mixed_attention_equals_sdpa_over_both_tiers(bits):
    cfg = S.CONFIGS["tiny"].scaled(hq=4, hkv=2, T=64, bits=bits, pct=25, recent=4)
    st, b, _ = _build(cfg, 23)
    qd, kd, vd = S.decode_tensors(cfg, 23, 0)
    N = cfg.T + 1
    o, p16, pq, st2 = O.decode_attention(st, N, qd, kd, vd, b)
    nq = N - cfg.cap16
    for g in range(2):
        Kq = O.dequantize_rows(st2["kq"][0, g, :nq], st2["ksz"][0, g, :nq], cfg.G, bits)
        Vq = O.dequantize_rows(st2["vq"][0, g, :nq], st2["vsz"][0, g, :nq], cfg.G, bits)
        K = np.concatenate([st2["k16"][0, g].astype(F64), Kq])
        V = np.concatenate([st2["v16"][0, g].astype(F64), Vq])
        for r in range(2):
            h = 2 * g + r
            ref = _sdpa(qd[0, h].astype(F64) / b[0, g].astype(F64), K, V)
            assert np.max(np.abs(o[0, h] - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
        # the new key is stored balanced, in the free slot
        s = st["free16"][0, g]
        assert np.array_equal(st2["k16"][0, g, s], (kd[0, g].astype(F32) * b[0, g]).astype(F16))
        # probability conservation: each query head distributes mass 1
        assert abs(p16[0, g].sum() + pq[0, g].sum() - 2.0) <= 1e-12


def test_permutation_invariance():
    """Attention is invariant under jointly permuting KV pairs (velog notes,
    section 3.4); the selection is by position, so it is invariant too."""
    cfg = S.CONFIGS["tiny"].scaled(hq=2, hkv=1, T=64, pct=25, recent=4)
    st, b, _ = _build(cfg, 31)
    qd, kd, vd = S.decode_tensors(cfg, 31, 0)
    N = cfg.T + 1
    o1, p1, st1, d1 = O.decode_step(st, N, qd, kd, vd, b, cfg.recent, cfg.H)
    rng = np.random.default_rng(0)
    p16 = rng.permutation(cfg.cap16)
    nq = N - cfg.cap16
    pq = rng.permutation(nq)
    sp = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in st.items()}
    for name in ("k16", "v16", "pos16", "acc16"):
        sp[name][0, 0] = st[name][0, 0][p16]
    sp["free16"][0, 0] = int(np.nonzero(p16 == st["free16"][0, 0])[0][0])
    for name in ("kq", "vq", "ksz", "vsz", "posq"):
        sp[name][0, 0, :nq] = st[name][0, 0, :nq][pq]
    o2, p2, st2, d2 = O.decode_step(sp, N, qd, kd, vd, b, cfg.recent, cfg.H)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    np.testing.assert_allclose(p2[0, 0], p1[0, 0][p16], atol=1e-15)
    assert st1["pos16"][0, 0, d1[0, 0]] == st2["pos16"][0, 0, d2[0, 0]]


def test_uniform_low_bit_case():
    """Importance budget 0: every cached token is low-bit; the new token is
    the only FP16 entry and is demoted right after its step."""
    cfg = S.CONFIGS["tiny"].scaled(T=32, pct=0, recent=0)
    st, b, _ = _build(cfg, 41)
    assert cfg.cap16 == 1
    N = cfg.T + 1
    qd, kd, vd = S.decode_tensors(cfg, 41, 0)
    o, p16, st2, drop = O.decode_step(st, N, qd, kd, vd, b, 0, 0)
    assert drop[0, 0] == 0 and st2["posq"][0, 0, N - 1] == N - 1
    Kq = O.dequantize_rows(st["kq"][0, 0, :N - 1], st["ksz"][0, 0, :N - 1], cfg.G, cfg.bits)
    Vq = O.dequantize_rows(st["vq"][0, 0, :N - 1], st["vsz"][0, 0, :N - 1], cfg.G, cfg.bits)
    kb_new = (kd[0, 0].astype(F32) * b[0, 0]).astype(F16).astype(F64)
    K = np.concatenate([kb_new[None], Kq])
    V = np.concatenate([vd[0, 0].astype(F64)[None], Vq])
    ref = _sdpa(qd[0, 0].astype(F64) / b[0, 0].astype(F64), K, V)
    assert np.max(np.abs(o[0, 0] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_multi_step_bookkeeping():
    cfg = S.CONFIGS["tiny"]
    st, b, _ = _build(cfg, 1000)
    N = cfg.T
    for step in range(8):
        N += 1
        qd, kd, vd = S.decode_tensors(cfg, 1000, step)
        _, _, st, drop = O.decode_step(st, N, qd, kd, vd, b, cfg.recent, cfg.H)
        live16 = np.delete(st["pos16"][0, 0], st["free16"][0, 0])
        live = np.concatenate([live16, st["posq"][0, 0, :N - cfg.B]])
        assert sorted(live.tolist()) == list(range(N))
        assert set(range(N - cfg.recent, N)) <= set(live16.tolist())


# ---------------------------------------------------------------- CriticalKV
def test_projected_l1_closed_forms():
    rng = np.random.default_rng(3)
    H, T, d = 3, 5, 4
    # W_O = identity: V_i W_O,h puts V_i in columns h*d..h*d+d-1 -> ||V_i||_1
    V = rng.standard_normal((H, T, d)).astype(F16)
    n1 = O.projected_value_l1(V, np.eye(H * d, dtype=F16))
    np.testing.assert_array_equal(n1, np.abs(V.astype(F64)).sum(axis=2))
    # V rows = unit vectors e_c: n_i = L1 norm of row h*d + c of W_O
    W = rng.standard_normal((H * d, 7)).astype(F16)
    c = rng.integers(0, d, (H, T))
    Ve = np.zeros((H, T, d), F16)
    for h in range(H):
        Ve[h, np.arange(T), c[h]] = 1
    n2 = O.projected_value_l1(Ve, W)
    for h in range(H):
        np.testing.assert_array_equal(n2[h], np.abs(W.astype(F64)[h * d + c[h]]).sum(axis=1))


def test_criticalkv_alpha_one_is_top_attention():
    rng = np.random.default_rng(8)
    H, T, d = 2, 30, 4
    A = (rng.integers(0, 6, (H, T)) / 8).astype(F32)
    V = rng.standard_normal((H, T, d)).astype(F16)
    W = rng.standard_normal((H * d, 5)).astype(F16)
    idx, score2, s1 = O.criticalkv_select(A, V, W, 9, 1.0)
    for h in range(H):
        assert idx[h].tolist() == sorted(O.top_by_key(A[h], np.arange(T), 9).tolist())
        assert s1[h].sum() == 9


def test_criticalkv_constant_norm_reduces_to_attention():
    """Equal ||V_i W_O||_1 for all i: stage 2 ranks by A alone, so the whole
    selection is the top-budget by attention weight."""
    rng = np.random.default_rng(9)
    H, T, d = 2, 40, 4
    A = rng.random((H, T)).astype(F32)
    V = np.zeros((H, T, d), F16)
    V[:, :, 0] = np.where(rng.random((H, T)) < 0.5, -2.0, 2.0)
    W = rng.standard_normal((H * d, 6)).astype(F16)
    for alpha in (0.0, 0.3, 0.5, 1.0):
        idx, _, _ = O.criticalkv_select(A, V, W, 11, alpha)
        for h in range(H):
            assert idx[h].tolist() == sorted(np.argsort(-A[h].astype(F64), kind="stable")[:11].tolist())


@pytest.mark.parametrize("seed", range(4))
def test_criticalkv_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    H, T, d = 1, int(rng.integers(3, 9)), 4
    A = (rng.integers(0, 4, (H, T)) / 4).astype(F32)
    V = np.zeros((H, T, d), F16)
    V[0, np.arange(T), rng.integers(0, d, T)] = rng.integers(1, 3, T)   # n_i closed form
    W = rng.integers(-2, 3, (H * d, 3)).astype(F16)
    n = np.array([np.abs(W.astype(F64)[np.nonzero(V[0, i])[0][0]]).sum() * float(V[0, i].max())
                  for i in range(T)])
    budget = int(rng.integers(1, T + 1))
    alpha = float(rng.choice([0.0, 0.5, 1.0]))
    b1 = int(math.floor(alpha * budget))
    idx, _, s1 = O.criticalkv_select(A, V, W, budget, alpha)
    S1 = _brute_top(A[0].astype(F64), np.arange(T), b1)
    rest = [i for i in range(T) if i not in S1]
    sc = (A[0].astype(F64) * n)[rest]
    S2 = [rest[j] for j in _brute_top(sc, np.array(rest), budget - b1)]
    assert idx[0].tolist() == sorted(S1 + S2)
    assert sorted(np.nonzero(s1[0])[0].tolist()) == S1


def test_criticalkv_stage1_mass_closed_form():
    """For softmax of N(0, s^2) logits, the top fraction f of entries carries
    mass ~ Phi(s - Phi^-1(1 - f)); with s = 3, f = 0.1 this is ~0.957 > 0.5,
    the stage-1 condition stated for CriticalKV (gist CriticalKV, Algorithm 1)."""
    from scipy.stats import norm
    cfg = S.CKV_CONFIGS["criticalkv_32k"]
    A, _, _ = S.criticalkv_inputs(dataclass_replace(cfg, H=2, hidden=8), 5)
    b1 = int(math.floor(cfg.alpha * cfg.budget))
    expect = norm.cdf(cfg.sigma - norm.ppf(1 - b1 / cfg.T))
    for h in range(2):
        top = O.top_by_key(A[h], np.arange(cfg.T), b1)
        mass = float(A[h].astype(F64)[top].sum())
        assert mass > 0.5 and abs(mass - expect) < 0.03


def dataclass_replace(cfg, **kw):
    import dataclasses
    return dataclasses.replace(cfg, **kw)


# ---------------------------------------------------------------- prefill scores (acc0)
def test_prefill_scores_conservation_and_single_token():
    """Every query row of a causal softmax sums to 1, so the scores of a
    group sum to rep * T; with one token each head gives it weight 1."""
    rng = np.random.default_rng(31)
    n, hq, hkv, T, d = 2, 6, 2, 37, 16
    q = rng.normal(0, 2, (n, hq, T, d)).astype(F16)
    k = rng.normal(0, 2, (n, hkv, T, d)).astype(F16)
    acc = O.prefill_scores(q, k)
    assert acc.shape == (n, hkv, T)
    assert np.allclose(acc.sum(axis=-1), hq // hkv * T, rtol=0, atol=1e-9)
    one = O.prefill_scores(q[:, :, :1], k[:, :, :1])
    assert np.allclose(one, hq // hkv, rtol=0, atol=1e-12)


def test_prefill_scores_zero_query_harmonic_tail():
    """q = 0 makes every causal row uniform: query i gives 1/(i+1) to each
    t <= i, so acc0[t] = rep * sum_{i=t}^{T-1} 1/(i+1)."""
    n, hq, hkv, T, d = 1, 4, 1, 50, 8
    q = np.zeros((n, hq, T, d), F16)
    k = np.random.default_rng(2).normal(size=(n, hkv, T, d)).astype(F16)
    acc = O.prefill_scores(q, k)
    tail = np.array([sum(1.0 / (i + 1) for i in range(t, T)) for t in range(T)])
    assert np.allclose(acc[0, 0], 4 * tail, rtol=1e-12, atol=0)


def test_prefill_scores_match_causal_sdpa_weights():
    """With the identity matrix as values, causal scaled-dot-product
    attention (torch, float64) returns the weight matrix itself; its column
    sums over the group's heads are acc0."""
    rng = np.random.default_rng(5)
    n, hq, hkv, T, d = 2, 8, 2, 29, 32
    q = rng.normal(0, 1.5, (n, hq, T, d)).astype(F16)
    k = rng.normal(0, 1.5, (n, hkv, T, d)).astype(F16)
    rep = hq // hkv
    qt = torch.from_numpy(q.astype(F64))
    kt = torch.from_numpy(np.repeat(k.astype(F64), rep, axis=1))
    eye = torch.eye(T, dtype=torch.float64).expand(n, hq, T, T)
    w = torch.nn.functional.scaled_dot_product_attention(qt, kt, eye, is_causal=True).numpy()
    ref = w.sum(axis=2).reshape(n, hkv, rep, T).sum(axis=2)
    assert np.allclose(O.prefill_scores(q, k), ref, rtol=1e-10, atol=1e-12)



# ---------------------------------------------------------------- multi-step H2O bookkeeping
def _grid_history(seed, T, steps, d, G, rep):
    """Keys whose per-token groups quantize losslessly at INT4: every group is
    z + 0.25*c with integer c in [0, 15] and both c = 0 and c = 15 present, so
    scale = 0.25 and zero = z exactly and dequant(quant(k)) == k. The mixed
    attention then equals plain softmax attention over the full history,
    whichever tokens sit in which tier, so the probabilities each step hands
    out can be recomputed from the history alone."""
    rng = np.random.default_rng(seed)
    n_tok = T + steps
    c = rng.integers(0, 16, (n_tok, d // G, G))
    c[:, :, 0] = 0
    c[:, :, 1] = 15
    for t in range(n_tok):
        for j in range(d // G):
            c[t, j] = c[t, j][rng.permutation(G)]
    z = rng.integers(-8, 9, (n_tok, d // G, 1)) * 0.25
    k_all = (z + 0.25 * c).reshape(n_tok, d).astype(F16)
    v_all = rng.standard_normal((n_tok, d)).astype(F16)
    q_all = (rng.standard_normal((steps, rep, d)) * 0.6).astype(F16)
    return k_all, v_all, q_all


def _brute_probs(q_all, k_all, T, j):
    """Softmax weights of decode step j (length T + j + 1) summed over the
    group's query heads, float64, from the full history (no tiers)."""
    N = T + j + 1
    d = k_all.shape[1]
    s = q_all[j].astype(F64) @ k_all[:N].astype(F64).T / math.sqrt(d)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).sum(axis=0)


def test_h2o_scores_carry_over_steps_and_restart_for_new_tokens():
    """acc after k decode steps = acc0 (prompt tokens) + the sum of every
    step's probability since the token arrived, recomputed from the history;
    a token appended during decode starts from 0, not from the score of the
    token it replaced in its slot (heavy hitters = accumulated attention,
    paperlayer section 5; the new token's score starts with its first step).
    Also re-runs the one-way selection from those brute-force scores: each
    step demotes the FP16 candidate outside the window with the smallest
    (score, -position), and its key and value rows land in the low-bit tier
    within scale/2 of the original rows."""
    T, steps, d, G, rep, B, R = 24, 7, 16, 8, 2, 10, 3
    H = B - R
    k_all, v_all, q_all = _grid_history(77, T, steps, d, G, rep)
    rng = np.random.default_rng(5)
    acc0 = (rng.integers(1, 6, T) * 0.125).astype(F32)[None, None]   # positive, with ties
    st = O.prefill_build(k_all[None, None, :T], v_all[None, None, :T], acc0, B, R, G, 4, T - B + steps)
    b = np.ones((1, 1, d), F32)
    bf = {int(p): F64(acc0[0, 0, p]) for p in st["pos16"][0, 0, :B]}     # brute-force scores
    resident = set(bf)
    demoted_kv_differ = False
    for j in range(steps):
        N = T + j + 1
        qd = q_all[j][None]
        kd, vd = k_all[N - 1][None, None], v_all[N - 1][None, None]
        _, _, st, drop = O.decode_step(st, N, qd, kd, vd, b, R, H)
        P = _brute_probs(q_all, k_all, T, j)
        bf[N - 1] = F64(0.0)
        resident.add(N - 1)
        for p in resident:
            bf[p] += P[p]
        cand = [p for p in resident if p < N - R]
        worst = min(cand, key=lambda p: (bf[p], -p))
        ranked = sorted(bf[p] for p in cand)
        assert ranked[1] - ranked[0] > 1e-6, "planted scores must not nearly tie"
        slot = N - (B + 1)
        dpos = int(st["posq"][0, 0, slot])
        assert dpos == worst, f"step {j}: demoted {dpos}, brute force {worst}"
        resident.remove(worst)
        # every resident token's stored score equals its brute-force sum
        pos16 = st["pos16"][0, 0]
        fr = st["free16"][0, 0]
        for s_ in range(B + 1):
            if s_ == fr:
                continue
            p = int(pos16[s_])
            assert p in resident
            assert abs(F64(st["acc16"][0, 0, s_]) - bf[p]) <= 1e-6 * max(1.0, bf[p]), (j, p)
        # the demoted rows: keys exact (grid), values within scale/2 of v
        kr = O.dequantize_rows(st["kq"][0, 0, slot:slot + 1], st["ksz"][0, 0, slot:slot + 1], G, 4)[0]
        assert np.array_equal(kr, k_all[dpos].astype(F64))
        vr = O.dequantize_rows(st["vq"][0, 0, slot:slot + 1], st["vsz"][0, 0, slot:slot + 1], G, 4)[0]
        vs = np.repeat(st["vsz"][0, 0, slot, :, 0].astype(F64), G)
        assert np.all(np.abs(vr - v_all[dpos].astype(F64)) <= 0.5 * vs * (1 + 1e-6))
        demoted_kv_differ |= not np.array_equal(st["vq"][0, 0, slot], st["kq"][0, 0, slot])
    assert demoted_kv_differ


def test_new_token_score_is_its_own_probability():
    """Right after its first step, the appended token's score is exactly the
    probability the group's heads gave it at that step (no carried score)."""
    T, d, G, rep, B, R = 20, 16, 8, 2, 8, 2
    k_all, v_all, q_all = _grid_history(3, T, 3, d, G, rep)
    acc0 = np.full((1, 1, T), 2.0, F32)
    st = O.prefill_build(k_all[None, None, :T], v_all[None, None, :T], acc0, B, R, G, 4, T - B + 3)
    b = np.ones((1, 1, d), F32)
    for j in range(3):
        N = T + j + 1
        fr = int(st["free16"][0, 0])
        _, _, st, _ = O.decode_step(st, N, q_all[j][None], k_all[N - 1][None, None],
                                    v_all[N - 1][None, None], b, R, B - R)
        assert st["pos16"][0, 0, fr] == N - 1
        P = _brute_probs(q_all, k_all, T, j)
        assert abs(F64(st["acc16"][0, 0, fr]) - P[N - 1]) <= 1e-6 * P[N - 1]


# ---------------------------------------------------------------- reduced-precision importance tier
def _grid_rows(rng, rows, d, G, bits):
    """Rows whose every group of G channels is z + s*c with integer c in
    [0, 2^bits - 1], c = 0 and c = 2^bits - 1 present, s a power of two and z
    a multiple of s: quantizing them at `bits` is lossless (scale s, zero z,
    codes c), and so is rebuilding them in fp16."""
    qmax = (1 << bits) - 1
    step = {8: 2.0 ** -4, 4: 0.25, 2: 1.0}[bits]
    c = rng.integers(0, qmax + 1, (rows, d // G, G))
    c[:, :, 0] = 0
    c[:, :, 1] = qmax
    for r in range(rows):
        for j in range(d // G):
            c[r, j] = c[r, j][rng.permutation(G)]
    z = rng.integers(-32, 33, (rows, d // G, 1)) * step
    return (z + step * c).reshape(rows, d).astype(F16)


@pytest.mark.parametrize("imp_bits,bits", [(8, 2), (4, 2), (8, 4)])
def test_importance_tier_on_lossless_rows_equals_fp16_tier(imp_bits, bits):
    """Importance tier quantized at imp_bits ([velog notes] Key contributions
    3), [paperlayer] section 3.3) on rows that imp_bits codes hold exactly:
    every step (attention output, probabilities, accumulated scores,
    selections, demoted codes) equals the fp16-tier oracle's, which the pins
    above tie to the pages. Prompt and new tokens are all grid rows; b = 1."""
    rng = np.random.default_rng(imp_bits * 10 + bits)
    n, hkv, rep, d, G, T, B, R, steps = 2, 2, 2, 16, 8, 30, 9, 3, 6
    ntok = T + steps
    k = np.stack([np.stack([_grid_rows(rng, ntok, d, G, imp_bits) for _ in range(hkv)]) for _ in range(n)])
    v = np.stack([np.stack([_grid_rows(rng, ntok, d, G, imp_bits) for _ in range(hkv)]) for _ in range(n)])
    q = (rng.standard_normal((steps, n, hkv * rep, d)) * 0.3).astype(F16)
    acc0 = (rng.integers(1, 6, (n, hkv, T)) * 0.125).astype(F32)
    b = np.ones((n, hkv, d), F32)
    capq = T - B + steps
    ref = O.prefill_build(k[:, :, :T], v[:, :, :T], acc0, B, R, G, bits, capq)
    imp = O.prefill_build(k[:, :, :T], v[:, :, :T], acc0, B, R, G, bits, capq, imp_bits=imp_bits)
    for i in range(n):
        for g in range(hkv):
            ki = O.dequantize_rows(imp["kimp"][i, g], imp["kimpsz"][i, g], G, imp_bits)
            assert np.array_equal(ki[:B], ref["k16"][i, g, :B].astype(F64))
    for j in range(steps):
        N = T + j + 1
        kd, vd = k[:, :, N - 1], v[:, :, N - 1]
        o1, p1, ref, d1 = O.decode_step(ref, N, q[j], kd, vd, b, R, B - R)
        o2, p2, imp, d2 = O.decode_step(imp, N, q[j], kd, vd, b, R, B - R)
        assert np.max(np.abs(o1 - o2)) <= 1e-12 * np.max(np.abs(o1))
        assert np.max(np.abs(p1 - p2)) <= 1e-12
        assert np.array_equal(d1, d2)
        for key in ("acc16", "pos16", "free16", "posq", "kq", "vq", "ksz", "vsz"):
            assert np.array_equal(np.asarray(ref[key]).view(np.uint8), np.asarray(imp[key]).view(np.uint8)), key


def test_importance_tier_new_token_and_demotion_bounds():
    """Random rows: a token in an 8-bit importance tier is held within
    scale/2 of its fp16 row, and once demoted its 2-bit codes hold it within
    the retained scale/2 plus that first error (plus one fp16 rounding):
    the demotion re-quantizes the same token's importance row, key and value
    each from their own row."""
    cfg = S.CONFIGS["tiny"].scaled(hq=2, hkv=1, T=64, pct=25, recent=4, bits=2)
    q, k, v, acc0 = S.prefill_tensors(cfg, 9)
    b, kb = O.balance(q, k)
    st = O.prefill_build(kb, v, acc0, cfg.B, cfg.recent, cfg.G, 2, cfg.capq(), imp_bits=8)
    G = cfg.G
    for step in range(6):
        N = cfg.T + step + 1
        qd, kd, vd = S.decode_tensors(cfg, 9, step)
        fr = int(st["free16"][0, 0])
        _, _, st, drop = O.decode_step(st, N, qd, kd, vd, b, cfg.recent, cfg.H)
        # the new token, quantized on arrival into the freed slot
        krow = (kd[0, 0].astype(F32) * b[0, 0]).astype(F16).astype(F64)
        ki = O.dequantize_rows(st["kimp"][0, 0, fr:fr + 1], st["kimpsz"][0, 0, fr:fr + 1], G, 8)[0]
        ks = np.repeat(st["kimpsz"][0, 0, fr, :, 0].astype(F64), G)
        assert np.all(np.abs(ki - krow) <= 0.5 * ks * (1 + 1e-6))
        vi = O.dequantize_rows(st["vimp"][0, 0, fr:fr + 1], st["vimpsz"][0, 0, fr:fr + 1], G, 8)[0]
        vsc = np.repeat(st["vimpsz"][0, 0, fr, :, 0].astype(F64), G)
        assert np.all(np.abs(vi - vd[0, 0].astype(F64)) <= 0.5 * vsc * (1 + 1e-6))
        # the demoted token: retained 2-bit codes around its importance row
        slot = N - cfg.cap16
        pos = int(st["posq"][0, 0, slot])
        src = kb if pos < cfg.T else None
        for name, arr in (("k", "kq"), ("v", "vq")):
            r = O.dequantize_rows(st[arr][0, 0, slot:slot + 1], st[arr[0] + "sz"][0, 0, slot:slot + 1], G, 2)[0]
            rs = np.repeat(st[arr[0] + "sz"][0, 0, slot, :, 0].astype(F64), G)
            if pos < cfg.T:
                orig = (kb if name == "k" else v)[0, 0, pos].astype(F64)
            else:
                kd2, vd2 = S.decode_tensors(cfg, 9, pos - cfg.T)[1:]
                orig = ((kd2[0, 0].astype(F32) * b[0, 0]).astype(F16) if name == "k" else vd2[0, 0]).astype(F64)
            # importance-tier error (8-bit scale over the group's range) + 2-bit
            # rounding + one fp16 rounding of the rebuilt row
            span = np.repeat((rs * 3.0).reshape(-1, 1), 1, axis=0)
            assert np.all(np.abs(r - orig) <= 0.5 * rs + span / 255.0 + 1e-3 * np.abs(orig) + 1e-6), (step, name)


# ---------------------------------------------------------------- output perturbation
def _pert_inputs(seed, H=3, T=40, d=8, hidden=12):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, d)).astype(F16)
    K = rng.standard_normal((H, T, d)).astype(F16)
    V = rng.standard_normal((H, T, d)).astype(F16)
    W = (rng.standard_normal((H * d, hidden)) * 0.3).astype(F16)
    return q, K, V, W


def test_perturbation_keep_all_and_single_token():
    """Keeping every token leaves the output unchanged (L = 0); keeping one
    token i makes the renormalised output exactly V_i, and o is the
    textbook attention (float64 SDPA)."""
    q, K, V, W = _pert_inputs(1)
    H, T, d = K.shape
    o, oh, Lh, Lp = O.output_perturbation(q, K, V, W, keep=[np.arange(T)] * H)
    assert np.all(Lh == 0) and np.all(Lp == 0)
    for h in range(H):
        assert np.max(np.abs(o[h] - _sdpa(q[h].astype(F64), K[h].astype(F64), V[h].astype(F64)))) <= 1e-12
    keep = [np.array([h * 5 + 2]) for h in range(H)]
    o, oh, Lh, Lp = O.output_perturbation(q, K, V, W, keep=keep)
    for h in range(H):
        i = keep[h][0]
        assert np.array_equal(oh[h], V[h, i].astype(F64))
        assert abs(Lh[h] - np.abs(o[h] - V[h, i].astype(F64)).sum()) <= 1e-12


def test_perturbation_projection_uses_the_heads_rows():
    """W_O made of per-head blocks c_h * I: the projected perturbation of head
    h is c_h times its head-space perturbation (a wrong row offset picks
    another head's c)."""
    q, K, V, _ = _pert_inputs(2, H=4, d=8)
    H, T, d = K.shape
    c = np.array([0.5, 2.0, 3.0, 0.25])
    W = np.zeros((H * d, H * d), F16)
    for h in range(H):
        W[h * d:(h + 1) * d, h * d:(h + 1) * d] = np.eye(d) * c[h]
    rng = np.random.default_rng(0)
    keep = [np.sort(rng.choice(T, 7, replace=False)) for _ in range(H)]
    _, _, Lh, Lp = O.output_perturbation(q, K, V, W, keep=keep)
    assert np.allclose(Lp, c * Lh, rtol=1e-12, atol=0)
    assert np.all(Lh > 0)


@pytest.mark.parametrize("seed", range(4))
def test_perturbation_within_its_attention_value_bound(seed):
    """The bound that ties the perturbation to A and V W_O: with u_i = V_i W_O,h,
    A the softmax weights and Z = sum of A over the kept set S,
      o - o_hat = sum_{i not in S} A_i u_i - (1/Z - 1) sum_{i in S} A_i u_i,
    so ||o - o_hat||_1 <= sum_{i not in S} A_i ||u_i||_1 + (1/Z - 1) sum_{i in S} A_i ||u_i||_1
    (triangle inequality; gist CriticalKV, theoretical framework). Also
    identical value rows give no perturbation whatever is kept."""
    q, K, V, W = _pert_inputs(10 + seed)
    H, T, d = K.shape
    rng = np.random.default_rng(seed)
    keep = [np.sort(rng.choice(T, int(rng.integers(1, T)), replace=False)) for _ in range(H)]
    _, _, _, Lp = O.output_perturbation(q, K, V, W, keep=keep)
    for h in range(H):
        s = (K[h].astype(F64) @ q[h].astype(F64)) / np.sqrt(d)
        A = np.exp(s - s.max())
        A /= A.sum()
        un = np.abs(V[h].astype(F64) @ W[h * d:(h + 1) * d].astype(F64)).sum(axis=1)
        S_ = np.zeros(T, bool)
        S_[keep[h]] = True
        Z = A[S_].sum()
        theta = (A[~S_] * un[~S_]).sum() + (1 / Z - 1) * (A[S_] * un[S_]).sum()
        assert Lp[h] <= theta * (1 + 1e-12)
    Vc = np.repeat(V[:, :1], T, axis=1)
    _, _, Lh, Lp = O.output_perturbation(q, K, Vc, W, keep=keep)
    assert np.all(Lh <= 1e-12) and np.all(Lp <= 1e-12)


def test_perturbation_of_a_given_output():
    """With o_hat given (a compressed cache's output) L is its distance to
    the full attention, e.g. 0 for the full attention itself."""
    q, K, V, W = _pert_inputs(3)
    o, _, _, _ = O.output_perturbation(q, K, V, W, keep=[np.arange(K.shape[1])] * K.shape[0])
    _, oh, Lh, Lp = O.output_perturbation(q, K, V, W, o_hat=o)
    assert np.array_equal(oh, o) and np.all(Lh == 0) and np.all(Lp == 0)
    _, _, Lh2, _ = O.output_perturbation(q, K, V, W, o_hat=o + 0.5)
    assert np.allclose(Lh2, 0.5 * K.shape[2], rtol=1e-12)
    # the projection is taken before the absolute value: an offset (+t, -t,
    # 0, ...) against an all-ones output column cancels exactly
    H, _, d = K.shape
    off = np.zeros((H, d))
    off[:, 0], off[:, 1] = 0.25, -0.25
    ones = np.ones((H * d, 1), F16)
    _, _, Lh3, Lp3 = O.output_perturbation(q, K, V, ones, o_hat=o + off)
    assert np.allclose(Lh3, 0.5, rtol=1e-12) and np.all(Lp3 <= 1e-12)


# ------------------------------------------------ per-channel key quantization
def _channel_grid_tile(rng, t, d, bits):
    """A tile whose every channel c is z_c + s_c * code with integer codes in
    [0, 2^bits - 1], 0 and 2^bits - 1 both present, s_c a power of two that
    differs widely between channels (outlier channels have large s_c) and z_c
    a multiple of s_c. Returns (x fp16, codes, s, z)."""
    qmax = (1 << bits) - 1
    e = rng.integers(-6, 4, d)
    e[[1, d // 2 + 3]] = 6                    # two outlier channels
    s = 2.0 ** e
    z = rng.integers(-8, 9, d) * s
    c = rng.integers(0, qmax + 1, (t, d))
    for ch in range(d):
        r0, r1 = rng.choice(t, 2, replace=False)
        c[r0, ch], c[r1, ch] = 0, qmax
    x = z[None, :] + c * s[None, :]
    assert np.array_equal(x.astype(F16).astype(F64), x)
    return x.astype(F16), c, s, z


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("d", [16, 128])
def test_channel_quantizer_lossless_grid(bits, d):
    """[velog notes] appendix C summary and [paperlayer] appendix C: keys
    quantized per channel over groups of 64 tokens. A tile built from known
    per-channel (scale, zero, codes) comes back exactly: each channel gets its
    own scale and zero (a per-token group, or channels mixed up, would not:
    the scales differ by up to 2^12 between channels)."""
    rng = np.random.default_rng(100 + bits + d)
    x, c, s, z = _channel_grid_tile(rng, O.KEY_TILE, d, bits)
    packed, sz = O.quantize_channels(x, bits)
    assert packed.shape == (O.KEY_TILE, d * bits // 8) and sz.shape == (d, 2)
    assert np.array_equal(O.unpack_codes(packed, d, bits), c)
    assert np.array_equal(sz[:, 0].astype(F64), s) and np.array_equal(sz[:, 1].astype(F64), z)
    assert np.array_equal(O.dequantize_channels(packed, sz, bits), x.astype(F64))
    # the per-token rule on the same tile is lossy: the pin tells them apart
    pt, szt = O.quantize_rows(x, d // 2, bits)
    assert not np.array_equal(O.dequantize_rows(pt, szt, d // 2, bits), x.astype(F64))


@pytest.mark.parametrize("bits", [4, 2])
def test_channel_quantizer_bound_and_outlier_isolation(bits):
    """Random tile with two outlier channels (x20, the synthetic outlier
    factor): every element is within s_c/2 of its channel's grid (plus the
    clamp term when the fp16 scale rounds down), and on the ordinary channels
    the per-channel error stays far below the per-token (group d/2) error,
    the isolation of outliers the appendix C summary credits it with."""
    rng = np.random.default_rng(7 + bits)
    t, d = O.KEY_TILE, 128
    x = rng.standard_normal((t, d))
    out = [5, 77]
    x[:, out] *= 20
    x = x.astype(F16)
    packed, sz = O.quantize_channels(x, bits)
    xr = O.dequantize_channels(packed, sz, bits)
    qmax = (1 << bits) - 1
    x64 = x.astype(F64)
    s = sz[:, 0].astype(F64)
    s_true = (x64.max(axis=0) - x64.min(axis=0)) / qmax
    bound = 0.5 * s + qmax * np.maximum(0.0, s_true - s) + 1e-6 * (np.abs(x64).max(axis=0) + s)
    err = np.abs(xr - x64)
    assert np.all(err <= bound[None, :])
    assert np.array_equal(O.unpack_codes(packed, d, bits)[x64.argmin(axis=0), np.arange(d)], np.zeros(d))
    pt, szt = O.quantize_rows(x, d // 2, bits)
    err_tok = np.abs(O.dequantize_rows(pt, szt, d // 2, bits) - x64)
    ordinary = np.setdiff1d(np.arange(d), out)
    assert err[:, ordinary].max() < 0.25 * err_tok[:, ordinary].max()


def _two_level_keys(rng, n, hkv, ntok, d, G, bits):
    """Keys whose every group j of G channels takes, in every token, only the
    values z_j and z_j + qmax * s_j (s_j a power of two): both the per-token
    group quantizer and the per-channel tile quantizer hold them exactly,
    whichever tokens share a tile (one level present: scale 0, zero = that
    level; both: scale s_j, codes 0 and qmax)."""
    qmax = (1 << bits) - 1
    s = 2.0 ** rng.integers(-4, 2, (n, hkv, 1, d // G, 1))
    z = rng.integers(-4, 5, (n, hkv, 1, d // G, 1)) * s
    hi = rng.random((n, hkv, ntok, d // G, G)) < 0.5
    return (z + hi * qmax * s).reshape(n, hkv, ntok, d).astype(F16)


@pytest.mark.parametrize("bits", [4, 2])
def test_key_tiles_on_lossless_keys_equal_per_token_cache(bits):
    """Per-channel key tiles with the fp16 buffer, on keys both quantizers hold
    exactly and values on the per-token grid: every decode step (output,
    probabilities, accumulated scores, selections) is bit-identical to the
    per-token cache's, which the pins above tie to the pages; the retained
    positions in tile order then buffer order are the per-token cache's slot
    order (demotion order), and the tiles' value codes are its rows. The
    prompt leaves 130 = 2*64 + 2 retained tokens, so the buffer starts with
    two pairs and fills (one tile flushed) at the 62nd step."""
    rng = np.random.default_rng(40 + bits)
    n, hkv, rep, d, G, T, B, R, steps = 1, 2, 2, 16, 8, 150, 20, 4, 70
    ntok = T + steps
    k = _two_level_keys(rng, n, hkv, ntok, d, G, bits)
    v = np.stack([np.stack([_grid_rows(rng, ntok, d, G, bits) for _ in range(hkv)]) for _ in range(n)])
    q = (rng.standard_normal((steps, n, hkv * rep, d)) * 0.3).astype(F16)
    acc0 = (rng.integers(1, 6, (n, hkv, T)) * 0.125).astype(F32)
    b = np.ones((n, hkv, d), F32)
    capq = 256
    ref = O.prefill_build(k[:, :, :T], v[:, :, :T], acc0, B, R, G, bits, capq)
    kt = O.prefill_build(k[:, :, :T], v[:, :, :T], acc0, B, R, G, bits, capq, key_tile=O.KEY_TILE)
    flushed = False
    for j in range(steps):
        N = T + j + 1
        kd, vd = k[:, :, N - 1], v[:, :, N - 1]
        o1, p1, ref, d1 = O.decode_step(ref, N, q[j], kd, vd, b, R, B - R)
        o2, p2, kt, d2 = O.decode_step(kt, N, q[j], kd, vd, b, R, B - R)
        assert np.array_equal(o1, o2) and np.array_equal(p1, p2)
        assert np.array_equal(d1, d2)
        for key in ("acc16", "pos16", "free16"):
            assert np.array_equal(ref[key], kt[key]), key
        D = N - B                                  # retained after this step
        nq, nb = O.retained_counts(kt, D)
        assert nq + nb == D and nb == (T - B + j + 1) % 64
        flushed |= nq == 192
        for i in range(n):
            for g in range(hkv):
                order = np.concatenate([kt["posq"][i, g, :nq], kt["posbuf"][i, g, :nb]])
                assert np.array_equal(order, ref["posq"][i, g, :D])
                assert np.array_equal(kt["vq"][i, g, :nq], ref["vq"][i, g, :nq])
                assert np.array_equal(kt["vsz"][i, g, :nq].view(np.uint16), ref["vsz"][i, g, :nq].view(np.uint16))
    assert flushed


def test_key_tiles_hold_the_history_rows():
    """Random balanced keys (outlier channels) through prefill and 75 decode
    steps with per-channel tiles: after every step the importance tier, the
    tiles and the buffer partition positions 0..N-1; the retained positions
    in tile then buffer order are the prompt's retained positions ascending
    followed by the decode steps' dropped positions in the order dropped;
    every tile is the per-channel quantization of its 64 positions' balanced
    keys (values per token) taken from the token history, and the buffer
    holds those rows in fp16. The step's attention output is softmax
    attention over exactly those keys and values (scaled-dot-product
    attention in float64)."""
    cfg = S.CONFIGS["tiny"].scaled(hq=2, hkv=1, T=120, pct=20, recent=4, bits=4)
    q, k, v, acc0 = S.prefill_tensors(cfg, 31)
    b, kb = O.balance(q, k)
    steps, KT, d = 75, O.KEY_TILE, cfg.d
    capq = 192
    st = O.prefill_build(kb, v, acc0, cfg.B, cfg.recent, cfg.G, cfg.bits, capq, key_tile=KT)
    hist_k = [kb[0, 0, t] for t in range(cfg.T)]
    hist_v = [v[0, 0, t] for t in range(cfg.T)]
    keep = set(st["pos16"][0, 0, :cfg.B].tolist())
    order = [t for t in range(cfg.T) if t not in keep]
    for j in range(steps):
        N = cfg.T + j + 1
        qd, kd, vd = S.decode_tensors(cfg, 31, j)
        hist_k.append(O.balance_keys(kd[0, 0], b[0, 0]))
        hist_v.append(vd[0, 0])
        before = st
        o, _, st, drop = O.decode_step(st, N, qd, kd, vd, b, cfg.recent, cfg.H)
        # the attention of this step, from the cache before it and the history
        nq, nb = O.retained_counts(before, N - cfg.B - 1)
        Kl, Vl = [], []
        held = np.arange(cfg.cap16) != before["free16"][0, 0]      # the free slot is stale
        for t in list(before["pos16"][0, 0][held]) + [N - 1]:
            Kl.append(hist_k[t].astype(F64))
            Vl.append(hist_v[t].astype(F64))
        for tj in range(nq // KT):
            tp = before["posq"][0, 0, tj * KT:(tj + 1) * KT]
            pk, szk = O.quantize_channels(np.stack([hist_k[t] for t in tp]), cfg.bits)
            Kl.extend(O.dequantize_channels(pk, szk, cfg.bits))
            pv, szv = O.quantize_rows(np.stack([hist_v[t] for t in tp]), cfg.G, cfg.bits)
            Vl.extend(O.dequantize_rows(pv, szv, cfg.G, cfg.bits))
        for t in before["posbuf"][0, 0, :nb]:
            Kl.append(hist_k[t].astype(F64))
            Vl.append(hist_v[t].astype(F64))
        assert len(Kl) == N
        for h in range(cfg.hq):
            qh = qd[0, h].astype(F64) / b[0, 0].astype(F64)
            ref = _sdpa(qh, np.stack(Kl), np.stack(Vl))
            assert np.max(np.abs(o[0, h] - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
        order.append(int(before["pos16"][0, 0, drop[0, 0]]) if drop[0, 0] != before["free16"][0, 0]
                     else N - 1)
        D = N - cfg.B
        nq, nb = O.retained_counts(st, D)
        got = np.concatenate([st["posq"][0, 0, :nq], st["posbuf"][0, 0, :nb]])
        assert np.array_equal(got, np.array(order))
        imp = st["pos16"][0, 0][np.arange(cfg.cap16) != st["free16"][0, 0]]
        assert np.array_equal(np.sort(np.concatenate([imp, got])), np.arange(N))
        for tj in range(nq // KT):
            tp = st["posq"][0, 0, tj * KT:(tj + 1) * KT]
            pk, szk = O.quantize_channels(np.stack([hist_k[t] for t in tp]), cfg.bits)
            assert np.array_equal(st["kq"][0, 0, tj * KT:(tj + 1) * KT], pk)
            assert np.array_equal(st["kcsz"][0, 0, tj].view(np.uint16), szk.view(np.uint16))
            pv, szv = O.quantize_rows(np.stack([hist_v[t] for t in tp]), cfg.G, cfg.bits)
            assert np.array_equal(st["vq"][0, 0, tj * KT:(tj + 1) * KT], pv)
        for r, t in enumerate(st["posbuf"][0, 0, :nb]):
            assert np.array_equal(st["kbuf"][0, 0, r].view(np.uint16), hist_k[t].view(np.uint16))
            assert np.array_equal(st["vbuf"][0, 0, r].view(np.uint16), hist_v[t].view(np.uint16))
    assert O.retained_counts(st, cfg.T + steps - cfg.B)[0] >= 2 * KT
