"""Parity of the HIP path (through the C interface) with the CPU oracle.

Bit-exact: balancer b and balanced keys, quantization codes and (scale,
zero), important-set positions, demoted rows, top-k selections.
Tolerance (fp32 accumulation vs fp64 oracle): attention outputs and
accumulated scores, max|gpu - oracle| <= 2e-3 * max|oracle|.
Multi-step decode is checked in lockstep: each step starts the oracle from
the device state, so fp32 probabilities that underflow to exactly 0 (which
fp64 keeps distinct) cannot make the two selections drift apart.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_decode_amd import _lib as L
from mixed_precision_decode_amd import synth as S

pytestmark = pytest.mark.gpu
F16, F32, F64 = np.float16, np.float32, np.float64
TOL = 2e-3


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits16(a):
    return np.ascontiguousarray(a).view(np.uint16)


def assert_close(gpu, ref, what, floor=0.0):
    """max|gpu - ref| <= TOL * max|ref| + floor. `floor` covers only values
    fp32 cannot hold: probabilities below 2^-126 flush to 0 on the device
    while fp64 keeps them."""
    ref = np.asarray(ref, F64)
    err = np.max(np.abs(np.asarray(gpu, F64) - ref)) if ref.size else 0.0
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    assert err <= TOL * scale + floor, f"{what}: max err {err:.3e} > {TOL} * {scale:.3e} + {floor:.1e}"


def dims_of(cfg, capq=None):
    return L.Dims(batch=cfg.batch, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, group=cfg.G, bits=cfg.bits,
                  cap16=cfg.cap16, capq=cfg.capq() if capq is None else capq, imp_bits=cfg.imp_bits,
                  key_tile=cfg.key_tile)


# ---------------------------------------------------------------- quantize
@pytest.mark.parametrize("d,group,bits", [(128, 64, 4), (128, 64, 2), (128, 128, 4),
                                          (64, 32, 4), (64, 32, 2), (64, 64, 2)])
@pytest.mark.parametrize("n_rows", [1, 37, 4099])
def test_quantize_parity(d, group, bits, n_rows):
    print(f"quantize d={d} G={group} bits={bits} rows={n_rows}", flush=True)
    rng = np.random.default_rng(n_rows * 7 + d + bits)
    x = rng.standard_normal((n_rows + 5, d)).astype(F32)
    x[:, rng.integers(0, d, 4)] *= 20
    x[::5] *= 1e-4            # fp16 subnormal territory
    x[::9] *= 300
    x = x.astype(F16)
    x[3 % len(x)] = F16(1.5)  # constant row
    x[4 % len(x), :group] = F16(-0.0)
    rows = rng.permutation(n_rows + 5)[:n_rows].astype(np.int32)
    for use_rows in (False, True):
        src = x[rows] if use_rows else x[:n_rows]
        codes = torch.zeros((n_rows, d * bits // 8), dtype=torch.uint8, device="cuda")
        sz = torch.zeros((n_rows, d // group, 2), dtype=torch.float16, device="cuda")
        L.mikv_quantize_tokens(dev(x), dev(rows) if use_rows else None, codes, sz, group, bits)
        ref_c, ref_sz = O.quantize_rows(src, group, bits)
        assert np.array_equal(host(codes), ref_c)
        assert np.array_equal(bits16(host(sz)), bits16(ref_sz))


def test_quantize_empty():
    codes = torch.zeros((0, 64), dtype=torch.uint8, device="cuda")
    sz = torch.zeros((0, 2, 2), dtype=torch.float16, device="cuda")
    x = torch.zeros((4, 128), dtype=torch.float16, device="cuda")
    L.mikv_quantize_tokens(x, None, codes, sz, 64, 4)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- balancer
def _balance_gpu(cfg, q, k, want_kb=True):
    dims = dims_of(cfg)
    T = q.shape[2]
    b = torch.empty((cfg.batch, cfg.hkv, cfg.d), dtype=torch.float32, device="cuda")
    kb = torch.empty(k.shape, dtype=torch.float16, device="cuda") if want_kb else None
    ws = torch.empty(max(1, L.mikv_balance_workspace(dims, T)), dtype=torch.uint8, device="cuda")
    L.mikv_balance_prefill(dims, T, dev(q), dev(k), b, kb, ws)
    return b, kb


@pytest.mark.parametrize("name,over", [
    ("tiny", {}), ("tiny", dict(T=1)), ("tiny", dict(T=0)),
    ("gqa_throughput", dict(batch=2, T=300)),
    ("llama2_7b_layer", dict(batch=1, hq=4, hkv=4, T=777)),
    ("llama3_8b_32k", dict(hq=8, hkv=2, T=5000)),
])
def test_balance_parity(name, over):
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"balance {name} {over}", flush=True)
    q, k, _, _ = S.prefill_tensors(cfg, 77)
    b, kb = _balance_gpu(cfg, q, k)
    rb, rkb = O.balance(q, k)
    assert np.array_equal(host(b).view(np.uint32), rb.view(np.uint32))
    if cfg.T > 0:
        assert np.array_equal(bits16(host(kb)), bits16(rkb))


# ---------------------------------------------------------------- prefill build
def _prefill_gpu(cfg, seed, balanced=True, capq=None, gpu_scores=False, edit=None):
    """Balancer and prefill build on the device. gpu_scores: the heavy-hitter
    scores acc0 come from the prompt through mikv_prefill_scores (the method's
    own chain) instead of the drawn stand-in; the returned acc0 is then the
    device's, which both sides consume. edit: (q, k, v) -> (q, k, v), applied
    to the drawn prompt before anything uses it."""
    q, k, v, acc0 = S.prefill_tensors(cfg, seed)
    if edit is not None:
        q, k, v = edit(q, k, v)
    dims = dims_of(cfg, capq)
    cache = L.Cache(dims)
    if balanced:
        b, _ = _balance_gpu(cfg, q, k, want_kb=False)
    else:
        b = torch.ones((cfg.batch, cfg.hkv, cfg.d), dtype=torch.float32, device="cuda")
    if gpu_scores:
        acc_d = torch.empty((cfg.batch, cfg.hkv, cfg.T), dtype=torch.float32, device="cuda")
        ws_s = torch.empty(max(1, L.mikv_prefill_scores_workspace(dims, cfg.T)), dtype=torch.uint8,
                           device="cuda")
        L.mikv_prefill_scores(dims, cfg.T, dev(q), dev(k), acc_d, ws_s)
        acc0 = host(acc_d)
    else:
        acc_d = dev(acc0)
    ws = torch.empty(max(1, L.mikv_h2o_workspace(dims, cfg.T)), dtype=torch.uint8, device="cuda")
    src = dict(k=dev(k), v=dev(v), acc0=acc_d, b=b if balanced else None)
    L.mikv_h2o_update_select(dims, cache, cfg.T, cfg.recent, cfg.H, src=src, ws=ws)
    return dims, cache, b, (q, k, v, acc0)


def _state_equal(gpu, ref):
    for key in ("pos16", "free16", "posq"):
        assert np.array_equal(gpu[key], ref[key]), key
    assert np.array_equal(gpu["acc16"].view(np.uint32), ref["acc16"].view(np.uint32))
    # fp16 importance rows or importance codes, whichever the cache holds;
    # per-channel key tiles and the fp16 buffer
    for key in ("k16", "v16", "ksz", "vsz", "kimpsz", "vimpsz", "kcsz", "kbuf", "vbuf"):
        if key in ref:
            assert np.array_equal(bits16(gpu[key]), bits16(ref[key])), key
    if "posbuf" in ref:
        assert np.array_equal(gpu["posbuf"], ref["posbuf"]), "posbuf"
    for key in ("kq", "vq", "kimp", "vimp"):
        if key in ref:
            assert np.array_equal(gpu[key], ref[key]), key


@pytest.mark.parametrize("name,over,balanced", [
    ("tiny", {}, True), ("tiny", {}, False),
    ("tiny", dict(pct=0, recent=0), True),          # uniform low-bit (B = 0)
    ("tiny", dict(pct=100, recent=16), True),       # everything important
    ("tiny", dict(recent=0), True),
    ("tiny", dict(recent=51), True),                # heavy = 0
    ("gqa_throughput", dict(batch=2, T=700), True),
    ("llama3_8b_32k", dict(hq=8, hkv=2, T=3000), True),
    # more rows than the scatter grid holds threads: rows loop with prefetch
    ("gqa_throughput", dict(batch=8, T=700), True),
    ("tiny", dict(batch=64, T=2500), True),
])
def test_prefill_build_parity(name, over, balanced):
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"prefill {name} {over} balanced={balanced}", flush=True)
    dims, cache, b, (q, k, v, acc0) = _prefill_gpu(cfg, 5, balanced)
    if balanced:
        _, kb = O.balance(q, k)
    else:
        kb = k
    ref = O.prefill_build(kb, v, acc0, cfg.B, cfg.recent, cfg.G, cfg.bits, cfg.capq(), imp_bits=cfg.imp_bits,
                           key_tile=cfg.key_tile)
    _state_equal(cache.to_numpy(), ref)


# ---------------------------------------------------------------- decode lockstep
def _units_state(cache, units):
    """The cache of the listed (sequence, kv head) units, gathered on the
    device and copied to the host, laid out as a batch of units with one kv
    head each (the oracle treats every unit independently)."""
    ns = torch.tensor([u[0] for u in units], device="cuda")
    gs = torch.tensor([u[1] for u in units], device="cuda")
    out = {k: getattr(cache, k)[ns, gs].unsqueeze(1).cpu().numpy() for k in cache.names}
    out["group"], out["bits"], out["imp_bits"] = cache.dims.group, cache.dims.bits, cache.imp_bits
    out["key_tile"] = cache.key_tile
    return out


def _units_inputs(cfg, units, qd, kd, vd, bh, o, p16, dpos):
    """Step inputs and device outputs of the listed units, in the same
    one-kv-head-per-unit layout."""
    r = cfg.rep
    q = np.stack([qd[n, g * r:(g + 1) * r] for n, g in units])
    k = np.stack([kd[n, g:g + 1] for n, g in units])
    v = np.stack([vd[n, g:g + 1] for n, g in units])
    b = np.stack([bh[n, g:g + 1] for n, g in units])
    oo = np.stack([o[n, g * r:(g + 1) * r] for n, g in units])
    pp = np.stack([p16[n, g:g + 1] for n, g in units])
    dp = np.stack([dpos[n, g:g + 1] for n, g in units])
    return q, k, v, b, oo, pp, dp


def _check_step(cfg, N, step, before, after, qd, kd, vd, bh, og, gp16, gdpos, mid=None):
    """One decode step of the device against the oracle started from the
    device's own state before the step (lockstep). All arrays are host
    arrays laid out [units or sequences][kv heads][...]."""
    ro, rp16, _, rst = O.decode_attention(before, N, qd, kd, vd, bh)
    if mid is not None:
        # separate calls: the attention call alone appends the new token
        for key in ("k16", "v16", "kimp", "vimp", "kimpsz", "vimpsz"):
            if key in rst:
                assert np.array_equal(np.asarray(mid[key]).view(np.uint8), np.asarray(rst[key]).view(np.uint8)), key
        assert np.array_equal(mid["pos16"], rst["pos16"])
    assert_close(og, ro, f"o step {step}")
    # probabilities below 2^-126 flush to 0 in fp32, fp64 keeps them
    underflow = N * cfg.rep * 2.0 ** -126
    assert_close(gp16.astype(F64), rp16, f"p16 step {step}", floor=underflow)
    acc_prev = before["acc16"].astype(F64)
    fr = before["free16"]
    for i in range(acc_prev.shape[0]):
        for g in range(acc_prev.shape[1]):
            acc_prev[i, g, fr[i, g]] = 0.0
    acc = after["acc16"].astype(F64)
    assert_close(acc, acc_prev + rp16, f"acc step {step}", floor=underflow)
    # the step's increment on its own, to the p16 rule; the stored fp32 sum
    # is rounded once (half an ulp of the new score)
    inc_err = np.abs(acc - acc_prev - rp16) - 2.0 ** -24 * np.abs(acc)
    lim = TOL * np.max(np.abs(rp16)) + underflow
    assert np.max(inc_err) <= lim, f"acc increment step {step}: {np.max(inc_err):.3e} > {lim:.3e}"
    # selection on the device's own fp32 scores must match exactly
    drop = O.select_drop(acc, rst["pos16"], N, cfg.recent, cfg.H)
    assert np.array_equal(after["free16"], drop), f"selection step {step}"
    ref_mid = dict(rst)
    ref_mid["acc16"] = after["acc16"]
    rdem = O.demote(ref_mid, N, drop)
    _state_equal(after, rdem)
    assert np.array_equal(gdpos, np.take_along_axis(rst["pos16"], drop[..., None], 2)[..., 0])


def _lockstep(cfg, seed, steps, balanced=True, check_every=1, fused=False, sample=0, gpu_scores=False, edit=None):
    """steps decode steps on the device; every check_every-th step (and the
    last) is compared with the oracle over all units, and with sample > 0
    every other step is compared over `sample` units (a different set each
    step). fused: one mikv_decode_step call per step (the benchmark's launch
    configuration); else mikv_decode_attn then mikv_h2o_update_select.
    gpu_scores: the prompt's heavy-hitter scores come from
    mikv_prefill_scores, and the prefill build on them is checked first."""
    dims, cache, b, (q, k, v, acc0) = _prefill_gpu(cfg, seed, balanced, gpu_scores=gpu_scores, edit=edit)
    bh = host(b)
    if gpu_scores:
        kb = O.balance(q, k)[1] if balanced else k
        ref = O.prefill_build(kb, v, acc0, cfg.B, cfg.recent, cfg.G, cfg.bits, cfg.capq(), imp_bits=cfg.imp_bits,
                           key_tile=cfg.key_tile)
        _state_equal(cache.to_numpy(), ref)
        print(f"  prefill build on the device's prompt scores matches the oracle", flush=True)
    del q, k, v
    o = torch.empty((cfg.batch, cfg.hq, cfg.d), dtype=torch.float32, device="cuda")
    p16 = torch.empty((cfg.batch, cfg.hkv, cfg.cap16), dtype=torch.float32, device="cuda")
    dpos = torch.empty((cfg.batch, cfg.hkv), dtype=torch.int32, device="cuda")
    ws = torch.zeros(L.mikv_decode_attn_workspace(dims, cfg.T + steps), dtype=torch.uint8,
                     device="cuda")
    n_units = cfg.batch * cfg.hkv
    N = cfg.T
    checked = sampled = 0
    for step in range(steps):
        N += 1
        qd, kd, vd = S.decode_tensors(cfg, seed, step)
        full = step % check_every == 0 or step == steps - 1
        units = None
        if not full and sample > 0:
            stride = max(1, n_units // sample)
            units = sorted({((step * 7 + j * stride) % n_units) for j in range(min(sample, n_units))})
            units = [(u // cfg.hkv, u % cfg.hkv) for u in units]
        before = cache.to_numpy() if full else (_units_state(cache, units) if units else None)
        mid = None
        if fused:
            L.mikv_decode_step(dims, cache, N, cfg.recent, cfg.H, dev(qd), dev(kd), dev(vd), b, o, p16,
                               ws, demoted_pos=dpos)
        else:
            L.mikv_decode_attn(dims, cache, N, dev(qd), dev(kd), dev(vd), b, o, p16, ws)
            if full:
                mid = cache.to_numpy()
            L.mikv_h2o_update_select(dims, cache, N, cfg.recent, cfg.H, p16=p16, demoted_pos=dpos)
        if full:
            _check_step(cfg, N, step, before, cache.to_numpy(), qd, kd, vd, bh, host(o), host(p16),
                        host(dpos), mid)
            checked += 1
            if check_every > 1:
                print(f"  step {step} (N={N}): all {n_units} units match the oracle", flush=True)
        elif units:
            ins = _units_inputs(cfg, units, qd, kd, vd, bh, host(o), host(p16), host(dpos))
            _check_step(cfg, N, step, before, _units_state(cache, units), *ins)
            sampled += 1
    return cache, checked, sampled


@pytest.mark.parametrize("name,over,balanced,steps", [
    ("tiny", {}, True, 32),
    ("tiny", {}, False, 32),
    ("tiny", dict(bits=2), True, 12),
    ("tiny", dict(pct=0, recent=0), True, 6),
    ("tiny", dict(pct=100, recent=16), True, 6),
    ("tiny", dict(recent=0), True, 6),
    ("tiny", dict(hq=4, hkv=1), True, 6),            # MQA-style group of 4
    ("tiny", dict(hq=8, hkv=1), True, 4),            # group of 8: two head tiles
    ("gqa_throughput", dict(batch=3, T=600), True, 5),
    ("llama3_8b_32k", dict(hq=8, hkv=2, T=4100), True, 4),
    ("llama3_8b_32k", dict(hq=8, hkv=4, T=3000), True, 3),   # two-head tiles of 2-bit codes
    ("gqa_throughput", dict(batch=2, hq=8, hkv=4, T=900), True, 3),  # two-head tiles of 4-bit codes
    ("tiny", dict(hq=6, hkv=1, T=300), True, 4),                      # three two-head tiles, ragged
    ("llama2_7b_layer", dict(batch=2, hq=3, hkv=3, T=1500), True, 4),
    # one (sequence, head) unit per 1024-thread block, whole units per block
    ("tiny", dict(batch=256), True, 6),
    ("tiny", dict(batch=512, bits=2), True, 4),                 # two units per block
    ("tiny", dict(batch=256, group=64, pct=0, recent=0), True, 3),
    ("llama2_7b_layer", dict(T=700), True, 3),
])
def test_decode_lockstep(name, over, balanced, steps):
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"lockstep {name} {over} balanced={balanced} steps={steps}", flush=True)
    _lockstep(cfg, 11, steps, balanced)


def _edge_rows(q, k, v):
    """Prompt rows at the edges of the code encodings: constant rows (scale
    0; a key row stays constant through the per-channel balancer only when it
    is zero), rows scaled into fp16's subnormal range (subnormal scales), wide
    value rows, and every other query head scaled down so that the low fp16
    parts of its q-hat are subnormals."""
    f32 = np.float32
    q, k, v = q.copy(), k.copy(), v.copy()
    k[:, :, 1::7] = k[:, :, 1::7, :1]
    k[:, :, 6::17] = 0
    v[:, :, 2::7] = v[:, :, 2::7, :1]
    k[:, :, 3::11] = (k[:, :, 3::11].astype(f32) * f32(1e-5)).astype(np.float16)
    v[:, :, 4::11] = (v[:, :, 4::11].astype(f32) * f32(1e-5)).astype(np.float16)
    v[:, :, 5::13] = (v[:, :, 5::13].astype(f32) * f32(64.0)).astype(np.float16)
    q[:, ::2] = (q[:, ::2].astype(f32) * f32(1e-2)).astype(np.float16)
    return q, k, v


@pytest.mark.parametrize("name,over,steps,balanced", [
    ("llama3_8b_32k", dict(hq=8, hkv=2, T=1500), 3, True),    # 2-bit codes, value sums on the matrix cores
    ("llama3_8b_32k", dict(hq=8, hkv=2, T=1500), 2, False),   # constant key rows kept constant
    ("llama3_8b_32k", dict(hq=8, hkv=4, T=1200), 3, True),    # the same with two-head tiles
    ("gqa_throughput", dict(batch=2, T=600), 3, True),        # 4-bit codes, vector value sums
    ("gqa_throughput", dict(batch=2, T=600), 2, False),
    ("tiny", dict(hq=4, hkv=1), 4, True),                     # head dim 64
    ("llama2_7b_layer", dict(batch=1, hq=2, hkv=2, T=700), 2, True),  # single-head tiles
])
def test_decode_lockstep_edge_rows(name, over, steps, balanced):
    """Lockstep decode (the fused step) over a prompt with constant,
    subnormal-scale and wide rows and small query heads: the codes enter the
    matrix cores as 1 + code * step and the constant part is taken back out
    through sums the matrix cores form themselves, which these rows stress."""
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"edge-row lockstep {name} {over} steps={steps} balanced={balanced}", flush=True)
    _lockstep(cfg, 23, steps, balanced, fused=True, edit=_edge_rows)


@pytest.mark.parametrize("name,over,steps", [
    ("tiny", {}, 16),
    ("tiny", dict(hq=8, hkv=2, bits=2), 8),
    # 1 sequence x 8 kv heads, groups of 4, INT2: the fused merge with a
    # separate p16/H2O block, decode_merge_kernel<128, 2, 8, true, 1>
    ("llama3_8b_32k", dict(T=6000), 4),
    # 43 x 8 units of 4 heads: 4 output groups per merge block and no room for
    # a separate H2O block (output block 0 runs it), <128, 4, 8, true, 4>
    ("gqa_throughput", dict(batch=43, T=400), 4),
    ("llama2_7b_layer", dict(T=700), 3),
])
def test_decode_lockstep_fused(name, over, steps):
    """mikv_decode_step (attention with the H2O update fused into its merge
    launch) against the oracle, every step."""
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"fused lockstep {name} {over} steps={steps}", flush=True)
    _lockstep(cfg, 13, steps, fused=True)


@pytest.mark.parametrize("name,over,steps", [
    ("tiny", dict(hq=4, hkv=2), 12),
    ("gqa_throughput", dict(batch=4, T=900), 6),
    ("llama2_7b_layer", {}, 12),
])
def test_prompt_scores_to_decode(name, over, steps):
    """The method's own chain: prompt heavy-hitter scores on the device
    (mikv_prefill_scores), the balancer and prefill build on those scores
    (exact against the oracle given the same scores), then decode steps
    through mikv_decode_step in lockstep with the oracle. The Llama-2-7B
    layer runs at full size (sampled units per step, all units at the last)."""
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"prompt scores -> prefill build -> decode: {name} {over} steps={steps}", flush=True)
    full = name == "llama2_7b_layer" and not over
    _lockstep(cfg, 1000 + list(S.CONFIGS).index(name), steps, fused=True, gpu_scores=True,
              check_every=steps if full else 1, sample=8 if full else 0)


# ---------------------------------------------------------------- reduced-precision importance tier
@pytest.mark.parametrize("name,over", [
    ("tiny", dict(imp_bits=8, bits=2)), ("tiny", dict(imp_bits=4, bits=2)),
    ("tiny", dict(imp_bits=8, bits=4, hq=4, hkv=2)), ("tiny", dict(imp_bits=4, bits=4, batch=64, T=700)),
    ("gqa_throughput", dict(batch=2, T=700, imp_bits=8, bits=2)),
    ("llama2_7b_layer", dict(batch=1, hq=4, hkv=4, T=900, imp_bits=4, bits=2)),
])
def test_prefill_build_importance_codes(name, over):
    """Prefill build with the importance tier stored as 8- or 4-bit codes:
    bit-exact against the oracle (importance and retained codes, scales,
    positions, scores)."""
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"prefill (importance codes) {name} {over}", flush=True)
    dims, cache, b, (q, k, v, acc0) = _prefill_gpu(cfg, 6, True)
    _, kb = O.balance(q, k)
    ref = O.prefill_build(kb, v, acc0, cfg.B, cfg.recent, cfg.G, cfg.bits, cfg.capq(), imp_bits=cfg.imp_bits,
                           key_tile=cfg.key_tile)
    _state_equal(cache.to_numpy(), ref)


@pytest.mark.parametrize("name,over,steps,fused", [
    ("tiny", dict(imp_bits=8, bits=2), 12, False),
    ("tiny", dict(imp_bits=4, bits=2), 12, True),
    ("tiny", dict(imp_bits=8, bits=4, hq=4, hkv=2), 8, True),      # two-head tiles
    ("tiny", dict(imp_bits=4, bits=2, hq=8, hkv=2), 8, False),     # four-head tiles
    ("tiny", dict(imp_bits=8, bits=2, hq=8, hkv=1), 4, True),      # two tiles of four heads
    ("tiny", dict(imp_bits=4, bits=4, recent=0), 6, True),
    ("tiny", dict(imp_bits=8, bits=2, pct=0, recent=0), 4, True),  # B = 0: only the new token
    ("gqa_throughput", dict(batch=3, T=600, imp_bits=8, bits=2), 4, True),
    ("llama3_8b_32k", dict(hq=8, hkv=2, T=4100, imp_bits=4, bits=2), 3, True),
    ("llama2_7b_layer", dict(batch=2, hq=3, hkv=3, T=1500, imp_bits=4, bits=2), 3, False),
    ("tiny", dict(imp_bits=4, bits=2, hq=3, hkv=1, batch=2, T=333), 6, True),  # three single-head tiles, ragged
    ("tiny", dict(imp_bits=4, bits=2, pct=0, recent=0), 4, False),             # B = 0: only the new token
    ("llama2_7b_layer", dict(batch=2, hq=2, hkv=2, T=2100, imp_bits=4, bits=4), 3, True),
])
def test_decode_lockstep_importance_codes(name, over, steps, fused):
    """Decode steps with an 8- or 4-bit importance tier against the oracle,
    every step: the new token quantized on append (exact codes), attention
    over both code tiers (tolerance), scores, selection and the demoted
    token re-quantized from its importance codes (exact)."""
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"lockstep (importance codes) {name} {over} steps={steps} fused={fused}", flush=True)
    _lockstep(cfg, 17, steps, fused=fused)


@pytest.mark.parametrize("name", ["llama2_7b_imp4", "llama2_7b_imp8"])
def test_decode_importance_codes_full_size(name):
    """The reduced-precision importance workloads at full size (8 x 32 heads,
    4096 tokens, 20% importance at INT4 / INT8, INT2 retention) through
    mikv_decode_step: 24 steps, all units at the first and last, 8 units at
    the others."""
    cfg = S.CONFIGS[name]
    print(f"full-size lockstep {name}", flush=True)
    _, checked, sampled = _lockstep(cfg, 1000 + list(S.CONFIGS).index(name), 24, check_every=23,
                                    fused=True, sample=8)
    assert checked + sampled == 24


# ---------------------------------------------------------------- per-channel key tiles
@pytest.mark.parametrize("name,over,balanced", [
    ("tiny", dict(key_tile=64), True),                            # 205 retained: 3 tiles + 13 buffered
    ("tiny", dict(key_tile=64), False),
    ("tiny", dict(key_tile=64, pct=0, recent=0), True),           # all 256 retained: 4 tiles, no buffer
    ("tiny", dict(key_tile=64, T=40, recent=4), True),            # 32 retained: buffer only
    ("tiny", dict(key_tile=64, bits=2, T=512, pct=25, recent=8, group=64), True),
    ("gqa_throughput", dict(key_tile=64, batch=2, T=700), True),
    ("llama2_7b_kchan", dict(batch=2, T=1000), True),
    ("llama3_8b_32k", dict(key_tile=64, hq=8, hkv=2, T=3000), True),
])
def test_prefill_build_key_tiles(name, over, balanced):
    """Prefill build with per-channel key tiles: tiles (codes and per-channel
    scale and zero), per-token value codes, buffered fp16 pairs and every
    position bit-exact against the oracle."""
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"prefill (key tiles) {name} {over} balanced={balanced}", flush=True)
    dims, cache, b, (q, k, v, acc0) = _prefill_gpu(cfg, 8, balanced)
    kb = O.balance(q, k)[1] if balanced else k
    ref = O.prefill_build(kb, v, acc0, cfg.B, cfg.recent, cfg.G, cfg.bits, cfg.capq(), key_tile=64)
    _state_equal(cache.to_numpy(), ref)


@pytest.mark.parametrize("name,over,steps,fused", [
    ("tiny", dict(key_tile=64), 80, False),                        # a tile flushed at step 51
    ("tiny", dict(key_tile=64, hq=8, hkv=2), 70, True),            # four-head tiles
    ("tiny", dict(key_tile=64, hq=4, hkv=2, bits=2), 70, True),    # two-head tiles
    ("tiny", dict(key_tile=64, T=40, recent=4), 100, True),        # first tile formed while decoding
    ("tiny", dict(key_tile=64, pct=0, recent=0), 70, False),       # B = 0
    ("tiny", dict(key_tile=64, batch=3, hq=6, hkv=3, group=64, bits=2), 66, True),
    ("gqa_throughput", dict(key_tile=64, batch=3, T=700), 70, True),
    ("llama3_8b_32k", dict(key_tile=64, hq=8, hkv=2, T=3000), 66, True),
    ("llama2_7b_kchan", dict(batch=2, hq=4, hkv=4, T=1000), 66, False),
])
def test_decode_lockstep_key_tiles(name, over, steps, fused):
    """Decode with per-channel key tiles against the oracle at every step:
    attention over the FP16 tier, the tiles and the buffered pairs
    (tolerance), scores and selection, the demoted pair in its buffer row and
    every flush of a full buffer into a tile (exact)."""
    cfg = S.CONFIGS[name].scaled(**over, steps=steps)   # capq holds every step
    print(f"lockstep (key tiles) {name} {over} steps={steps} fused={fused}", flush=True)
    _lockstep(cfg, 19, steps, fused=fused)


def test_decode_key_tiles_full_size():
    """The per-channel key-tile workload at full size (8 x 32 heads, 4096
    tokens, 20% importance, INT4) through mikv_decode_step over all 128
    steps: all units every 32nd step and at the last (those include flushes
    of every unit's buffer), 8 units at the others."""
    cfg = S.CONFIGS["llama2_7b_kchan"]
    print(f"full-size lockstep {cfg.name}", flush=True)
    _, checked, sampled = _lockstep(cfg, 1000 + list(S.CONFIGS).index(cfg.name), cfg.steps, check_every=32,
                                    fused=True, sample=8)
    assert checked + sampled == cfg.steps


@pytest.mark.parametrize("name,check_every", [("llama2_7b_layer", 16), ("llama3_8b_32k", 8),
                                              ("gqa_throughput", 20)])
def test_decode_full_size(name, check_every):
    """The configs' full shapes over every decode step they define, through
    mikv_decode_step as the benchmark launches it (seed 1000 + config index).
    Every step is compared with the oracle, started from the device state
    before that step: over all units every check_every-th step and at the
    last, over 8 units (a different set each step) at the others."""
    cfg = S.CONFIGS[name]
    print(f"full-size lockstep {name}: {cfg.steps} steps, all units every {check_every}", flush=True)
    _, checked, sampled = _lockstep(cfg, 1000 + list(S.CONFIGS).index(name), cfg.steps,
                                    check_every=check_every, fused=True, sample=8)
    assert checked + sampled == cfg.steps
    print(f"full-size lockstep {name}: {checked} full checks, {sampled} sampled", flush=True)


# ---------------------------------------------------------------- CriticalKV
def _ckv_gpu(A, V, W, budget, alpha):
    H, T = A.shape
    idx = torch.empty((H, budget), dtype=torch.int32, device="cuda")
    sc = torch.empty((H, T), dtype=torch.float32, device="cuda")
    ws = torch.empty(L.mikv_criticalkv_workspace(H, T, V.shape[-1], W.shape[1]), dtype=torch.uint8,
                     device="cuda")
    L.mikv_criticalkv_select(dev(A), dev(V), dev(W), budget, alpha, idx, sc, ws)
    return host(idx), host(sc)


def _ckv_check(A, V, W, budget, alpha, sample=None):
    H, T = A.shape
    idx, sc = _ckv_gpu(A, V, W, budget, alpha)
    b1 = int(np.floor(F64(alpha) * budget))
    pos = np.arange(T)
    s1 = np.zeros((H, T), bool)
    for h in range(H):
        s1[h, O.top_by_key(A[h], pos, b1)] = True
    assert np.array_equal(sc < 0, s1), "stage-1 membership"
    rng = np.random.default_rng(0)
    rows = []
    for h in range(H):
        rest = pos[~s1[h]]
        rows.append(rest if sample is None or len(rest) <= sample else np.sort(rng.choice(rest, sample, replace=False)))
    norms = O.projected_value_l1(V, W, rows=rows)
    for h in range(H):
        r = rows[h]
        assert_close(sc[h, r], A[h, r].astype(F64) * norms[h, r], f"score2 head {h}")
    ridx, _, _ = O.criticalkv_select(A, V, W, budget, alpha, score2=sc.astype(F64))
    assert np.array_equal(idx, ridx)
    if sample is None:
        # the oracle's own fp64 selection may differ from the device's only
        # at near-ties of its stage-2 score around the cutoff (counted)
        oidx, _, _ = O.criticalkv_select(A, V, W, budget, alpha)
        s64 = A.astype(F64) * O.projected_value_l1(V, W)
        b2 = budget - b1
        ties = 0
        for h in range(H):
            diff = np.setxor1d(idx[h], oidx[h])
            if len(diff) == 0:
                continue
            rest = pos[~s1[h]]
            cut = np.sort(s64[h, rest])[::-1][b2 - 1]
            gap = np.max(np.abs(s64[h, diff] - cut))
            assert gap <= TOL * np.max(s64[h, rest]), f"head {h}: selections differ away from the cutoff ({gap:.3e})"
            ties += len(diff) // 2
        print(f"criticalkv: {ties} near-tie swaps against the fp64 oracle over {H} heads", flush=True)


@pytest.mark.parametrize("H,T,hidden,budget,alpha", [
    (8, 1000, 256, 200, 0.5), (8, 1000, 256, 200, 0.0), (8, 1000, 256, 200, 1.0),
    (3, 257, 128, 1, 0.5), (3, 257, 128, 257, 0.5), (16, 4099, 512, 811, 0.3),
    # decimals whose float32 rounding lies below the decimal: floor(0.7f * 10) = 6,
    # floor(0.7 * 10) = 7 in double
    (4, 300, 128, 10, 0.7), (4, 300, 128, 10, 0.9), (4, 1000, 128, 100, 0.29),
])
def test_criticalkv_parity(H, T, hidden, budget, alpha):
    print(f"criticalkv H={H} T={T} hidden={hidden} budget={budget} alpha={alpha}", flush=True)
    cfg = dataclasses.replace(S.CKV_CONFIGS["criticalkv_32k"], H=H, T=T, hidden=hidden)
    A, V, W = S.criticalkv_inputs(cfg, 3)
    _ckv_check(A, V, W, budget, alpha)


def test_criticalkv_full_size():
    cfg = S.CKV_CONFIGS["criticalkv_32k"]
    print("criticalkv full size", flush=True)
    A, V, W = S.criticalkv_inputs(cfg, 1004)
    _ckv_check(A, V, W, cfg.budget, cfg.alpha, sample=192)


# ---------------------------------------------------------------- graph replay
def test_graph_replay_matches_eager():
    """Decode steps captured as HIP graphs (one graph per step, as the
    benchmark replays them) give bit-identical caches and outputs to eager
    launches, with eager work and synchronisations between the replays."""
    cfg = S.CONFIGS["tiny"].scaled(hq=4, hkv=2)
    outs = []
    for use_graph in (False, True):
        dims, cache, b, _ = _prefill_gpu(cfg, 21, True)
        o = torch.zeros((cfg.batch, cfg.hq, cfg.d), dtype=torch.float32, device="cuda")
        p16 = torch.zeros((cfg.batch, cfg.hkv, cfg.cap16), dtype=torch.float32, device="cuda")
        ws = torch.zeros(L.mikv_decode_attn_workspace(dims, cfg.T + 6), dtype=torch.uint8, device="cuda")
        inputs = [tuple(dev(x) for x in S.decode_tensors(cfg, 21, s)) for s in range(6)]
        graphs = []
        if use_graph:
            for s in range(6):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    L.mikv_decode_attn(dims, cache, cfg.T + s + 1, *inputs[s], b, o, p16, ws)
                    L.mikv_h2o_update_select(dims, cache, cfg.T + s + 1, cfg.recent, cfg.H, p16=p16)
                graphs.append(g)
        trace = []
        for s in range(6):
            if use_graph:
                graphs[s].replay()
                torch.ones(1 << 20, device="cuda").sum()   # eager work between replays
            else:
                L.mikv_decode_attn(dims, cache, cfg.T + s + 1, *inputs[s], b, o, p16, ws)
                L.mikv_h2o_update_select(dims, cache, cfg.T + s + 1, cfg.recent, cfg.H, p16=p16)
            torch.cuda.synchronize()
            trace.append((host(o).copy(), host(p16).copy(), cache.to_numpy()))
        outs.append(trace)
    for (o1, p1, c1), (o2, p2, c2) in zip(*outs):
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
        assert np.array_equal(p1.view(np.uint32), p2.view(np.uint32))
        for key in L.Cache.NAMES:
            assert np.array_equal(np.asarray(c1[key]).view(np.uint8), np.asarray(c2[key]).view(np.uint8)), key


# ---------------------------------------------------------------- determinism
@pytest.mark.parametrize("name,over,steps", [
    ("llama3_8b_32k", dict(hq=8, hkv=2, T=6000), 3),   # head tiles, value sums on the matrix cores
    ("gqa_throughput", dict(batch=8, T=1500), 3),       # head tiles, 4-bit codes
    ("llama2_7b_layer", dict(batch=2, T=2000), 3),      # single-head splits
])
def test_runs_bit_identical(name, over, steps):
    """Two runs from the same prompt, prompt scores from mikv_prefill_scores
    included, give bit-identical prompt scores, outputs, probabilities and
    caches at every step: every reduction on the path has a fixed order."""
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"determinism {name} {over} steps={steps}", flush=True)
    runs = []
    for _ in range(2):
        dims, cache, b, (_, _, _, acc0) = _prefill_gpu(cfg, 31, True, gpu_scores=True)
        o = torch.zeros((cfg.batch, cfg.hq, cfg.d), dtype=torch.float32, device="cuda")
        p16 = torch.zeros((cfg.batch, cfg.hkv, cfg.cap16), dtype=torch.float32, device="cuda")
        dpos = torch.zeros((cfg.batch, cfg.hkv), dtype=torch.int32, device="cuda")
        ws = torch.zeros(L.mikv_decode_attn_workspace(dims, cfg.T + steps), dtype=torch.uint8, device="cuda")
        trace = [np.asarray(acc0).copy()]
        for step in range(steps):
            qd, kd, vd = S.decode_tensors(cfg, 31, step)
            L.mikv_decode_step(dims, cache, cfg.T + step + 1, cfg.recent, cfg.H, dev(qd), dev(kd), dev(vd), b,
                               o, p16, ws, demoted_pos=dpos)
            trace.append((host(o).copy(), host(p16).copy(), host(dpos).copy(), cache.to_numpy()))
        runs.append(trace)
    a, b2 = runs
    assert np.array_equal(a[0].view(np.uint32), b2[0].view(np.uint32)), "prompt scores"
    for step, ((o1, p1, d1, c1), (o2, p2, d2, c2)) in enumerate(zip(a[1:], b2[1:])):
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)), f"o step {step}"
        assert np.array_equal(p1.view(np.uint32), p2.view(np.uint32)), f"p16 step {step}"
        assert np.array_equal(d1, d2), f"demoted positions step {step}"
        for key in L.Cache.NAMES:
            assert np.array_equal(np.asarray(c1[key]).view(np.uint8), np.asarray(c2[key]).view(np.uint8)), \
                f"{key} step {step}"


# ---------------------------------------------------------------- fused decode step
@pytest.mark.parametrize("name,over,steps", [
    ("tiny", {}, 8), ("tiny", dict(hq=8, hkv=2, bits=2), 6), ("tiny", dict(recent=0), 4),
    ("tiny", dict(pct=0, recent=0), 4), ("tiny", dict(group=64), 4),
    ("gqa_throughput", dict(batch=2, T=900), 3),
    ("llama3_8b_32k", dict(hq=8, hkv=2, T=20000, pct=25), 2),    # FP16 tier > 4096 slots: unfused path
    ("tiny", dict(batch=256), 4), ("tiny", dict(batch=512, bits=2, group=64), 3),  # one-pass kernel
    ("llama2_7b_layer", dict(T=700), 2),
    # 1024 units: the merge grid is too large for a separate p16 / H2O block,
    # so output block 0 of each unit does that work after its outputs
    ("tiny", dict(batch=1024), 2),
])
def test_decode_step_matches_separate_calls(name, over, steps):
    """mikv_decode_step is bit-identical to mikv_decode_attn followed by
    mikv_h2o_update_select (decode mode)."""
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"decode_step {name} {over}", flush=True)
    runs = []
    for fused in (False, True):
        dims, cache, b, _ = _prefill_gpu(cfg, 31, True)
        o = torch.zeros((cfg.batch, cfg.hq, cfg.d), dtype=torch.float32, device="cuda")
        p16 = torch.zeros((cfg.batch, cfg.hkv, cfg.cap16), dtype=torch.float32, device="cuda")
        dpos = torch.zeros((cfg.batch, cfg.hkv), dtype=torch.int32, device="cuda")
        ws = torch.zeros(L.mikv_decode_attn_workspace(dims, cfg.T + steps), dtype=torch.uint8, device="cuda")
        trace = []
        for s in range(steps):
            N = cfg.T + s + 1
            qd, kd, vd = (dev(x) for x in S.decode_tensors(cfg, 31, s))
            if fused:
                L.mikv_decode_step(dims, cache, N, cfg.recent, cfg.H, qd, kd, vd, b, o, p16, ws,
                                   demoted_pos=dpos)
            else:
                L.mikv_decode_attn(dims, cache, N, qd, kd, vd, b, o, p16, ws)
                L.mikv_h2o_update_select(dims, cache, N, cfg.recent, cfg.H, p16=p16, demoted_pos=dpos)
            trace.append((host(o).copy(), host(p16).copy(), host(dpos).copy(), cache.to_numpy()))
        runs.append(trace)
    for (o1, p1, d1, c1), (o2, p2, d2, c2) in zip(*runs):
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
        assert np.array_equal(p1.view(np.uint32), p2.view(np.uint32))
        assert np.array_equal(d1, d2)
        for key in L.Cache.NAMES:
            assert np.array_equal(np.asarray(c1[key]).view(np.uint8), np.asarray(c2[key]).view(np.uint8)), key


# ---------------------------------------------------------------- timed launch
@pytest.mark.parametrize("name,over", [("llama2_7b_layer", dict(T=700)), ("tiny", dict(hq=8, hkv=2))])
def test_decode_attn_timed_matches_plain(name, over):
    """mikv_decode_attn_timed computes exactly what mikv_decode_attn does
    and its events bracket the split kernel (a positive duration no longer
    than the whole call's)."""
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"decode_attn_timed {name} {over}", flush=True)
    res = []
    for timed in (False, True):
        dims, cache, b, _ = _prefill_gpu(cfg, 41, True)
        o = torch.zeros((cfg.batch, cfg.hq, cfg.d), dtype=torch.float32, device="cuda")
        p16 = torch.zeros((cfg.batch, cfg.hkv, cfg.cap16), dtype=torch.float32, device="cuda")
        ws = torch.zeros(L.mikv_decode_attn_workspace(dims, cfg.T + 1), dtype=torch.uint8, device="cuda")
        qd, kd, vd = (dev(x) for x in S.decode_tensors(cfg, 41, 0))
        if timed:
            e0, e1, c0, c1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
            c0.record()
            L.mikv_decode_attn_timed(dims, cache, cfg.T + 1, qd, kd, vd, b, o, p16, ws, e0, e1)
            c1.record()
            torch.cuda.synchronize()
            t_split, t_call = e0.elapsed_time(e1), c0.elapsed_time(c1)
            assert 0.0 < t_split <= t_call, (t_split, t_call)
        else:
            L.mikv_decode_attn(dims, cache, cfg.T + 1, qd, kd, vd, b, o, p16, ws)
        res.append((host(o).copy(), host(p16).copy(), cache.to_numpy()))
    (o1, p1, c1), (o2, p2, c2) = res
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(p1.view(np.uint32), p2.view(np.uint32))
    for key in L.Cache.NAMES:
        assert np.array_equal(np.asarray(c1[key]).view(np.uint8), np.asarray(c2[key]).view(np.uint8)), key


# ---------------------------------------------------------------- read probe
@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096 + 48, 7), (1 << 22, 1024), ((1 << 20) + 16 * 5, 4096)])
def test_read_probe_reads_every_word(nbytes, blocks):
    """The streaming-read probe (measurement helper) touches the whole
    buffer: the XOR of its per-block words equals the XOR of all words."""
    rng = np.random.default_rng(nbytes + blocks)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32).copy()).cuda()
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    L.mikv_read_probe(buf, blocks, sink)
    got = np.bitwise_xor.reduce(host(sink).view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


def test_quantize_golden_ties_on_device():
    """The hand-derived quantizer vectors (tests/golden), including exact
    half-integer quotients that round half to even, through the device
    quantizer. Each golden group's values are tiled over a 32-channel group
    of a d = 64 row (tiling keeps the group's min, max, scale and codes); the
    device codes and (scale, zero) must equal the golden ones."""
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quantizer_hand_vectors.json")))
    d, group = 64, 32
    for case in gold["cases"]:
        g, bits = case["group"], case["bits"]
        x = np.asarray(case["x"], F64).astype(F16).reshape(-1, g)
        codes = np.asarray(case["codes"], np.int64).reshape(-1, g)
        rows_x, rows_c, rows_sz = [], [], []
        for i in range(x.shape[0]):            # one device row per golden group: both halves hold it
            rows_x.append(np.tile(x[i], 2 * group // g))
            rows_c.append(np.tile(codes[i], 2 * group // g))
            rows_sz.append([[case["scale"][i], case["zero"][i]]] * 2)
        xr = np.stack(rows_x).astype(F16)
        out = torch.zeros((len(xr), d * bits // 8), dtype=torch.uint8, device="cuda")
        sz = torch.zeros((len(xr), d // group, 2), dtype=torch.float16, device="cuda")
        print(f"golden {case['name']}", flush=True)
        L.mikv_quantize_tokens(dev(xr), None, out, sz, group, bits)
        assert np.array_equal(O.unpack_codes(host(out), d, bits), np.stack(rows_c)), case["name"]
        assert np.array_equal(host(sz).astype(F64), np.asarray(rows_sz, F64)), case["name"]


# ---------------------------------------------------------------- free-running
@pytest.mark.parametrize("name,over,steps", [
    ("tiny", {}, 32),
    ("tiny", dict(batch=64, hq=4, hkv=2), 16),
    ("llama2_7b_layer", dict(batch=1, T=700), 8),
    ("gqa_throughput", dict(batch=2, T=600), 8),
])
def test_decode_free_running(name, over, steps):
    """Device decode steps (mikv_decode_step) and the oracle's, each from its
    own state after the same prefill. Per (sequence, kv head) unit, outputs
    match to tolerance and the demoted positions agree until the unit's first
    divergence; a divergence must be a near-tie (the two candidates' fp64
    scores within the tolerance of the accumulated scores), after which the
    unit's states differ and it is no longer compared."""
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"free-running {name} {over} steps={steps}", flush=True)
    dims, cache, b, _ = _prefill_gpu(cfg, 77, True)
    st = cache.to_numpy()
    bh = host(b)
    o = torch.empty((cfg.batch, cfg.hq, cfg.d), dtype=torch.float32, device="cuda")
    p16 = torch.empty((cfg.batch, cfg.hkv, cfg.cap16), dtype=torch.float32, device="cuda")
    dpos = torch.empty((cfg.batch, cfg.hkv), dtype=torch.int32, device="cuda")
    ws = torch.zeros(L.mikv_decode_attn_workspace(dims, cfg.T + steps), dtype=torch.uint8, device="cuda")
    live = np.ones((cfg.batch, cfg.hkv), bool)
    diverged = 0
    for step in range(steps):
        N = cfg.T + step + 1
        qd, kd, vd = S.decode_tensors(cfg, 77, step)
        L.mikv_decode_step(dims, cache, N, cfg.recent, cfg.H, dev(qd), dev(kd), dev(vd), b, o, p16, ws,
                           demoted_pos=dpos)
        ro, rp16, _, rst = O.decode_attention(st, N, qd, kd, vd, bh)
        acc = O.h2o_accumulate(rst["acc16"], rp16)
        rst["acc16"] = acc.astype(F32)
        drop = O.select_drop(acc, rst["pos16"], N, cfg.recent, cfg.H)
        og, dp = host(o), host(dpos)
        rpos = np.take_along_axis(rst["pos16"], drop[..., None], 2)[..., 0]
        floor = N * cfg.rep * 2.0 ** -126
        for i in range(cfg.batch):
            for g in range(cfg.hkv):
                if not live[i, g]:
                    continue
                hs = slice(g * cfg.rep, (g + 1) * cfg.rep)
                assert_close(og[i, hs], ro[i, hs], f"o step {step} unit ({i},{g})")
                if dp[i, g] != rpos[i, g]:
                    slot = np.nonzero(rst["pos16"][i, g] == dp[i, g])[0]
                    assert len(slot) == 1, f"step {step} unit ({i},{g}): demoted position {dp[i, g]} not resident"
                    gap = abs(acc[i, g, slot[0]] - acc[i, g, drop[i, g]])
                    assert gap <= TOL * np.max(acc[i, g]) + floor, \
                        f"step {step} unit ({i},{g}): selections differ by {gap:.3e}, not a near-tie"
                    live[i, g] = False
                    diverged += 1
        st = O.demote(rst, N, drop)
    print(f"free-running {name}: {diverged} of {live.size} units diverged over {steps} steps, "
          f"all at near-ties", flush=True)
