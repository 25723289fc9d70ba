"""Benchmark of the MiKV mixed-precision decode path on one MI355X.

A step is one decode step of the whole batch (mikv_decode_step):
mixed-precision attention over both cache tiers (append + scores + softmax +
value sum) and the H2O accumulate / re-select / demote, in two launches (the
attention's merge kernel also runs the H2O update). The cache is built once
before timing (balancer + prefill build on the GPU) from seeded synthetic
inputs; every step consumes a new seeded (q, k, v) token per sequence and
kv head, so the low-bit tier grows by one token per step.

Per decode workload: --steps timed steps after --warmup steps (mean and
median step time; `value` = KV-tokens/s over the timed steps), then
--attn-steps replays of one attention call (split + merge, events around the
call) and as many of the split kernel alone (events of its own launch,
mikv_decode_attn_timed); medians are reported. The headline line is the
Llama-2-7B-shaped layer; the 32K GQA layer and the GQA throughput batch
follow in the same run under "configs". The CPU baseline leg replays one
more step of sequence 0 on the oracle, timed on the host cores, and compares
its result with the device's ("parity").

Before each timed launch an untimed read of a 1 GiB device buffer evicts the
caches (MI355X has a 256 MB Infinity Cache, larger than the per-step working
set of the workloads), so each launch streams its cache from HBM. The flush
reads rather than writes: a written flush leaves the Infinity Cache full of
dirty lines whose write-back would then compete with the measured kernel
(--flush write shows that case, --flush none the warm-cache case). Times
come from HIP events recorded on the stream the kernels run on.

The JSON line's roofline is the dominant kernel's: the split kernel. Other
modes, one JSON line each: --prefill (balancer, prefill build, prompt
heavy-hitter scores), --quantize (mikv_quantize_tokens on every prompt row),
--criticalkv (the CriticalKV select, 32 heads x 32K tokens), --perturbation
(the output-perturbation diagnostic of H2O, CriticalKV and MiKV), --read-ceiling
(a plain streaming read of one split launch's bytes), --calibrate-copy (the
1 GiB copy that scales the HBM counters).

Prints one JSON line. --gpus N > 1 is refused: the path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "mixed-precision decode attn KV-tokens/s + achieved HBM GB/s (% of peak)"
HBM_PEAK_GBPS = 8000.0
# sources compiled into the decode-attention kernels; the HBM traffic recorded
# under profiles/ is reported only while their hash matches the recorded one
KERNEL_SOURCES = ("mixed_precision_decode_amd/csrc/decode_attn.hip",
                  "mixed_precision_decode_amd/csrc/decode_tile.hpp",
                  "mixed_precision_decode_amd/csrc/decode_tile_mv.hpp",
                  "mixed_precision_decode_amd/csrc/common.hpp",
                  "mixed_precision_decode_amd/csrc/kernels.hpp",
                  "mixed_precision_decode_amd/csrc/h2o_common.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_hbm_traffic.json")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def split_kernel_name(cfg):
    """The kernel of the split step for this cache, as the library picks it:
    tiles of 2-4 query heads (an even group) and caches whose importance tier
    holds codes run decode_tile_kernel when quantization groups are d/2 and
    keys are quantized per token; everything else runs decode_split_kernel."""
    rt = 4 if cfg.rep % 4 == 0 else (2 if cfg.rep % 2 == 0 else 1)
    tile = cfg.key_tile == 0 and cfg.G == cfg.d // 2 and (cfg.imp_bits < 16 or rt > 1)
    return "decode_tile_kernel" if tile else "decode_split_kernel"


def recorded_traffic(workload, key="split_traffic_bytes_per_launch"):
    """HBM bytes per launch of the split kernel (key
    split_traffic_bytes_per_launch) or per decode-attention call, split +
    merge (call_traffic_bytes), from the FETCH_SIZE / WRITE_SIZE counter runs
    recorded under profiles/, each scaled by the reading of a plain 1 GiB
    copy; None when the kernels changed since the counters were taken or the
    workload was not profiled."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    w = rec.get("workloads", {}).get(workload)
    return None if w is None or key not in w else float(w[key])


def imp_row_bytes(cfg):
    """Bytes of one importance-tier token, key and value: fp16 rows, or
    codes plus an fp16 (scale, zero) per group for a reduced-precision tier."""
    if cfg.imp_bits == 16:
        return 4 * cfg.d
    return 2 * (cfg.d * cfg.imp_bits // 8 + 4 * (cfg.d // cfg.G))


def retained_bytes(cfg, nr):
    """Bytes of nr retained tokens, keys and values. Per-token keys: codes
    plus an fp16 (scale, zero) per group, K and V. Per-channel key tiles:
    the whole tiles' key codes plus an fp16 (scale, zero) per channel and
    tile, value codes with their per-token groups, and the buffered pairs as
    fp16 rows."""
    d, G = cfg.d, cfg.G
    cb, vsz = d * cfg.bits // 8, 4 * (d // G)
    if not cfg.key_tile:
        return nr * 2 * (cb + vsz)
    nq, nb = nr // cfg.key_tile * cfg.key_tile, nr % cfg.key_tile
    return nq * (2 * cb + vsz) + (nq // cfg.key_tile) * 4 * d + nb * 4 * d


def attn_bytes(cfg, N):
    """Algorithmic bytes of one decode-attention launch at length N (new
    token included): importance-tier rows read (cap16-1), the new token read
    (k_new, v_new) and appended, the retained tokens (retained_bytes), q, b,
    o and p16."""
    d = cfg.d
    per_unit = ((cfg.cap16 - 1) * imp_row_bytes(cfg) + 4 * d + imp_row_bytes(cfg)
                + retained_bytes(cfg, N - cfg.cap16)
                + cfg.rep * d * 2 + d * 4 + cfg.rep * d * 4 + cfg.cap16 * 4)
    return per_unit * cfg.batch * cfg.hkv


def split_bytes(cfg, N):
    """Algorithmic bytes of one split-kernel launch at length N: everything
    attn_bytes counts except o and p16, which the merge kernel writes."""
    return attn_bytes(cfg, N) - (cfg.rep * cfg.d * 4 + cfg.cap16 * 4) * cfg.batch * cfg.hkv


def h2o_bytes(cfg):
    """acc16 read+write, p16 and pos16 read per importance slot; the demoted
    K/V rows read and written as codes (per-channel key tiles: written to the
    buffer as fp16 rows, and one step in 64 the buffer read and written back
    as a tile, counted here as its 1/64 share)."""
    d = cfg.d
    if cfg.key_tile:
        tile = cfg.key_tile * 4 * d + retained_bytes(cfg, cfg.key_tile)
        per_unit = cfg.cap16 * 16 + 8 * d + 16 + tile / cfg.key_tile
    else:
        per_unit = cfg.cap16 * 16 + imp_row_bytes(cfg) + 2 * (d * cfg.bits // 8 + 4 * (d // cfg.G)) + 16
    return per_unit * cfg.batch * cfg.hkv


def cpu_baseline(cfg, before, b_np, N, q_np, k_np, v_np, gpu, budget_s):
    """The CPU oracle (as it stands) on a bounded sample of the same workload:
    the decode step of sequence 0 (all its kv heads) from the device's state
    before that step, repeated until budget_s. The first repetition's result
    is also compared with what the device computed for the same step
    (returned under "parity"): o and the accumulated scores to the stated
    tolerance, the demoted token chosen from the device's own fp32 scores and
    its codes exactly, and whether the oracle's fp64 scores pick the same
    token."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    reps = 0
    t0 = time.perf_counter()
    c0 = time.process_time()
    first = None
    while True:
        res = O.decode_step(before, N, q_np, k_np, v_np, b_np, cfg.recent, cfg.H)
        if first is None:
            first = res
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    # cores actually used: the process's CPU time over the wall time (numpy's
    # elementwise work is single-threaded; only its BLAS calls use the pool)
    busy = (time.process_time() - c0) / el
    # parity of the device's step with the oracle's, on this sample
    o_ref, p16_ref, st_ref, drop_ref = first
    tol = 2e-3
    o_err = float(np.max(np.abs(gpu["o"].astype(np.float64) - o_ref)) / np.max(np.abs(o_ref)))
    acc_prev = before["acc16"].astype(np.float64).copy()
    for g in range(cfg.hkv):
        acc_prev[0, g, before["free16"][0, g]] = 0.0
    acc_ref = acc_prev + p16_ref
    acc_gpu = gpu["after"]["acc16"].astype(np.float64)
    acc_err = float(np.max(np.abs(acc_gpu - acc_ref)) / np.max(np.abs(acc_ref)))
    _, _, _, appended = O.decode_attention(before, N, q_np, k_np, v_np, b_np)
    drop_dev = O.select_drop(acc_gpu, appended["pos16"], N, cfg.recent, cfg.H)
    sel_ok = bool(np.array_equal(gpu["after"]["free16"], drop_dev))
    mid = dict(appended)
    mid["acc16"] = gpu["after"]["acc16"]
    dem = O.demote(mid, N, drop_dev)
    slot = N - cfg.cap16
    raw = lambda a: np.ascontiguousarray(np.asarray(a)[:, :, slot]).view(np.uint8)
    if cfg.key_tile:
        # the demoted pair's buffer row, and the tile when it filled the buffer
        full = lambda a: np.ascontiguousarray(np.asarray(a)).view(np.uint8)
        codes_ok = all(np.array_equal(full(gpu["after"][key]), full(dem[key]))
                       for key in ("kbuf", "vbuf", "posbuf", "kq", "vq", "kcsz", "vsz", "posq"))
    else:
        codes_ok = all(np.array_equal(raw(gpu["after"][key]), raw(dem[key]))
                       for key in ("kq", "vq", "ksz", "vsz", "posq"))
    parity = {"units": f"sequence 0, {cfg.hkv} kv heads, step N={N}",
              "o_max_err_rel": o_err, "acc_max_err_rel": acc_err, "tolerance": tol,
              "selection_on_device_scores_exact": sel_ok, "demoted_codes_exact": bool(codes_ok),
              "oracle_fp64_selection_agrees": bool(np.array_equal(drop_ref, drop_dev)),
              "ok": bool(o_err <= tol and acc_err <= tol and sel_ok and codes_ok)}
    return {"value": reps * N / el, "unit": "KV-tokens/s", "cores": max(1, int(round(busy))),
            "cores_busy": busy, "blas_threads": int(threads), "kind": "oracle",
            "sample": (f"{reps} oracle decode steps of 1 of {cfg.batch} sequences "
                       f"({cfg.hkv} kv heads, N={N}), fp64 numpy, {el:.1f} s; "
                       f"host os.cpu_count()={os.cpu_count()}"),
            "parity": parity}


def calibrate_copy(nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size: the reference kernel
    whose FETCH_SIZE / WRITE_SIZE readings scale the counters of the MiKV
    kernels."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ts = []
    for _ in range(reps):
        ev[0].record()
        dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
        ts.append(ev[0].elapsed_time(ev[1]))
    t = float(np.median(ts)) * 1e-3
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps,
                      "copy_GBps": 2 * nbytes / t / 1e9}), flush=True)


def bench_quantize(args, log):
    """mikv_quantize_tokens on every prompt row of the workload, keys and
    values (2 * batch * hkv * T rows of d fp16). HBM-bound: per row it reads
    2d bytes and writes d*bits/8 code bytes plus an fp16 (scale, zero) pair
    per group."""
    import torch
    from mixed_precision_decode_amd import _lib as L
    from mixed_precision_decode_amd import synth as S
    cfg = S.CONFIGS[args.workload]
    _, k, v, _ = S.prefill_tensors(cfg, args.seed)
    x = torch.from_numpy(np.ascontiguousarray(np.stack([k, v]).reshape(-1, cfg.d))).cuda()
    n_rows = x.shape[0]
    codes = torch.empty((n_rows, cfg.d * cfg.bits // 8), dtype=torch.uint8, device="cuda")
    sz = torch.empty((n_rows, cfg.d // cfg.G, 2), dtype=torch.float16, device="cuda")
    nbytes = n_rows * (2.0 * cfg.d + cfg.d * cfg.bits / 8 + 4.0 * cfg.d / cfg.G)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    fo = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        L.mikv_quantize_tokens(x, None, codes, sz, cfg.G, cfg.bits)
    evs = _events(args.steps)
    for e0, e1 in evs:
        torch.sum(flush, dim=0, out=fo)
        e0.record()
        L.mikv_quantize_tokens(x, None, codes, sz, cfg.G, cfg.bits)
        e1.record()
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3
    gbps = nbytes / (us * 1e-6) / 1e9
    log(f"[bench] quantize {n_rows} rows: {us:.1f} us, {gbps:.0f} GB/s")
    return {"metric": "quantize GB/s", "value": gbps, "unit": "GB/s", "higher_is_better": True,
            "steps": args.steps, "warmup": args.warmup, "dtype": "f32", "data": "synthetic",
            "config": {"workload": cfg.name, "rows": n_rows, "head_dim": cfg.d, "bits": cfg.bits,
                       "group": cfg.G},
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS, "bytes_per_launch": nbytes, "kernel_us": us,
                         "kernel": "quantize_rows_kernel"}}


def read_ceiling(args, log):
    """A plain streaming read (mikv_read_probe: 16-byte nontemporal loads,
    one contiguous chunk per block) of as many bytes as one split-kernel
    launch of the workload, timed like the decode kernels: 1 GiB read flush
    before each launch, HIP events on the stream. Grids of 1024 to 8192
    blocks are tried; the fastest is the practical HBM read ceiling the
    decode kernels are compared against, next to the 8 TB/s vendor peak."""
    import torch
    from mixed_precision_decode_amd import _lib as L
    from mixed_precision_decode_amd import synth as S
    cfg = S.CONFIGS[args.workload]
    nbytes = int(split_bytes(cfg, cfg.T + 1)) // 16 * 16
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    fo = torch.empty((), dtype=torch.float32, device="cuda")
    res = {}
    for blocks in (1024, 2048, 4096, 8192):
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
        for _ in range(args.warmup):
            L.mikv_read_probe(buf, blocks, sink)
        evs = _events(args.steps)
        for e0, e1 in evs:
            torch.sum(flush, dim=0, out=fo)
            e0.record()
            L.mikv_read_probe(buf, blocks, sink)
            e1.record()
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3
        res[blocks] = {"us": us, "GBps": nbytes / (us * 1e-6) / 1e9}
        log(f"[bench] streaming read of {nbytes / 1e6:.1f} MB, {blocks} blocks: {us:.1f} us, "
            f"{res[blocks]['GBps']:.0f} GB/s")
    best = max(res, key=lambda b: res[b]["GBps"])
    gbps = res[best]["GBps"]
    return {"metric": "streaming-read ceiling GB/s", "value": gbps, "unit": "GB/s", "higher_is_better": True,
            "steps": args.steps, "warmup": args.warmup, "bytes": nbytes, "best_blocks": best,
            "frac_of_peak": gbps / HBM_PEAK_GBPS, "kernel": "mikv_read_probe (plain 16-byte nontemporal reads)",
            "by_blocks": res, "config": {"workload": cfg.name}}


def _events(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def bench_criticalkv(args, log):
    """CriticalKV prefill select at 32 heads x 32K tokens (hidden 4096): the
    two-stage selection with the ||V_h W_O,h||_1 projection on MFMA. Flops
    are the projection's algorithmic 2 (T - b1) d hidden per head."""
    import torch
    from mixed_precision_decode_amd import _lib as L
    from mixed_precision_decode_amd import synth as S
    cfg = S.CKV_CONFIGS["criticalkv_32k"]
    A, V, W = S.criticalkv_inputs(cfg, args.seed)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    Ag, Vg, Wg = dev(A), dev(V), dev(W)
    budget = cfg.budget
    b1 = int(np.floor(np.float64(cfg.alpha) * budget))
    idx = torch.empty((cfg.H, budget), dtype=torch.int32, device="cuda")
    ws = torch.empty(L.mikv_criticalkv_workspace(cfg.H, cfg.T, cfg.d, cfg.hidden), dtype=torch.uint8,
                     device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    fo = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        L.mikv_criticalkv_select(Ag, Vg, Wg, budget, cfg.alpha, idx, ws=ws)
    evs = _events(args.steps)
    for e0, e1 in evs:
        torch.sum(flush, dim=0, out=fo)
        e0.record()
        L.mikv_criticalkv_select(Ag, Vg, Wg, budget, cfg.alpha, idx, ws=ws)
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    flops = 2.0 * (cfg.T - b1) * cfg.d * cfg.hidden * cfg.H
    log(f"[bench] criticalkv select {ms:.3f} ms, {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s over the call")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        h = 0
        t0 = time.perf_counter()
        c0 = time.process_time()
        O.criticalkv_select(A[h:h + 1], V[h:h + 1], W[h * cfg.d:(h + 1) * cfg.d], budget, cfg.alpha)
        el = time.perf_counter() - t0
        busy = (time.process_time() - c0) / el
        cpu = {"value": el * cfg.H * 1e3, "unit": "ms per select (32 heads, extrapolated)", "kind": "oracle",
               "cores": max(1, int(round(busy))), "cores_busy": busy,
               "sample": f"1 of {cfg.H} heads, fp64 numpy, {el:.1f} s"}
    return {"metric": "CriticalKV prefill select ms (MFMA projection TFLOP/s)", "value": ms, "unit": "ms",
            "higher_is_better": False, "steps": args.steps, "warmup": args.warmup, "dtype": "f16 MFMA, f32 accumulate",
            "data": "synthetic",
            "config": {"workload": cfg.name, "heads": cfg.H, "head_dim": cfg.d, "hidden": cfg.hidden,
                       "context": cfg.T, "budget": budget, "alpha": cfg.alpha},
            "roofline": {"bound": "mfma", "achieved": flops / (ms * 1e-3) / 1e12, "peak": 2500.0,
                         "unit": "TFLOP/s", "frac": flops / (ms * 1e-3) / 1e12 / 2500.0,
                         "flops_per_call": flops, "kernel": "mikv_criticalkv_select (stage 1 + W_O layout pass + projection + stage 2)"},
            "context": "the pages report about 0.06 s added TTFT at 32K, batch 1 (hardware not given)",
            "cpu_baseline": cpu}


def bench_perturbation(args, log):
    """Output-perturbation diagnostic (gist CriticalKV, theoretical framework)
    on one Llama-2-shaped layer at the CriticalKV page's 32K batch-1 setting:
    32 heads of 128 channels, 32768 prompt tokens plus one new token, W_O
    4096 wide, 20% budget. Kept sets: H2O (recent window + heavy hitters of
    the prompt's accumulated attention, the set MiKV keeps in fp16) and
    CriticalKV (two-stage, alpha 0.5, on the same scores); MiKV's own output
    (fp16 + INT4 cache). Times one mikv_output_perturbation call per method
    (HBM-bound: K and V of every head once, plus W_O)."""
    import torch
    from mixed_precision_decode_amd import _lib as L
    from mixed_precision_decode_amd import synth as S
    cfg = S.CONFIGS["llama2_7b_layer"].scaled(batch=1, T=32768)
    hidden, alpha = 4096, 0.5
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    t0 = time.perf_counter()
    q, k, v, _ = S.prefill_tensors(cfg, args.seed)
    dims = L.Dims(batch=1, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, group=cfg.G, bits=cfg.bits, cap16=cfg.cap16,
                  capq=cfg.capq())
    qg, kg, vg = dev(q), dev(k), dev(v)
    del q
    acc0 = torch.empty((1, cfg.hkv, cfg.T), dtype=torch.float32, device="cuda")
    ws_s = torch.empty(L.mikv_prefill_scores_workspace(dims, cfg.T), dtype=torch.uint8, device="cuda")
    L.mikv_prefill_scores(dims, cfg.T, qg, kg, acc0, ws_s)
    b = torch.empty((1, cfg.hkv, cfg.d), dtype=torch.float32, device="cuda")
    ws_b = torch.empty(L.mikv_balance_workspace(dims, cfg.T), dtype=torch.uint8, device="cuda")
    L.mikv_balance_prefill(dims, cfg.T, qg, kg, b, None, ws_b)
    del qg, ws_s, ws_b
    cache = L.Cache(dims)
    ws_h = torch.empty(L.mikv_h2o_workspace(dims, cfg.T), dtype=torch.uint8, device="cuda")
    L.mikv_h2o_update_select(dims, cache, cfg.T, cfg.recent, cfg.H, src=dict(k=kg, v=vg, acc0=acc0, b=b), ws=ws_h)
    qd, kd, vd = S.decode_tensors(cfg, args.seed, 0)
    o = torch.empty((1, cfg.hq, cfg.d), dtype=torch.float32, device="cuda")
    p16 = torch.empty((1, cfg.hkv, cfg.cap16), dtype=torch.float32, device="cuda")
    ws = torch.zeros(L.mikv_decode_attn_workspace(dims, cfg.T + 1), dtype=torch.uint8, device="cuda")
    L.mikv_decode_attn(dims, cache, cfg.T + 1, dev(qd), dev(kd), dev(vd), b, o, p16, ws)
    H, T, B, d = cfg.hq, cfg.T, cfg.B, cfg.d
    Kf = torch.cat([kg[0], dev(kd[0]).unsqueeze(1)], dim=1).contiguous()
    Vf = torch.cat([vg[0], dev(vd[0]).unsqueeze(1)], dim=1).contiguous()
    W = dev((np.random.default_rng(args.seed).standard_normal((H * d, hidden)) / np.sqrt(hidden)).astype(np.float16))
    keep_h2o = torch.sort(cache.pos16[0], dim=1).values.contiguous()
    idx = torch.empty((H, B), dtype=torch.int32, device="cuda")
    ws_c = torch.empty(L.mikv_criticalkv_workspace(H, T, d, hidden), dtype=torch.uint8, device="cuda")
    L.mikv_criticalkv_select(acc0[0], vg[0].contiguous(), W, B, alpha, idx, ws=ws_c)
    keep_ckv = torch.cat([idx, torch.full((H, 1), T, dtype=torch.int32, device="cuda")], dim=1).contiguous()
    o_mikv = o[0].contiguous()
    del kg, vg, cache, ws, ws_h, ws_c
    qq = dev(qd[0])
    wsp = torch.empty(L.mikv_perturbation_workspace(H, T + 1, d, hidden), dtype=torch.uint8, device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    fo = torch.empty((), dtype=torch.float32, device="cuda")
    log(f"[bench] perturbation inputs ready ({time.perf_counter() - t0:.1f}s)")
    res = {}
    nbytes = 2.0 * H * (T + 1) * d * 2 + H * d * hidden * 2 + H * d * 2
    for name, kw in (("h2o", dict(keep=keep_h2o)), ("criticalkv", dict(keep=keep_ckv)),
                     ("mikv", dict(o_hat=o_mikv))):
        Lh = torch.empty(H, dtype=torch.float32, device="cuda")
        Lp = torch.empty(H, dtype=torch.float32, device="cuda")
        call = lambda: L.mikv_output_perturbation(qq, Kf, Vf, W, Lh, Lp, wsp, **kw)
        for _ in range(args.warmup):
            call()
        evs = _events(args.steps)
        for e0, e1 in evs:
            torch.sum(flush, dim=0, out=fo)
            e0.record()
            call()
            e1.record()
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(e) for a, e in evs])) * 1e3
        res[name] = {"us": us, "GBps": nbytes / (us * 1e-6) / 1e9, "mean_L_proj": float(Lp.mean()),
                     "mean_L_head": float(Lh.mean()), "L_proj": Lp.cpu().numpy()}
        log(f"[bench] perturbation {name}: {us:.1f} us ({res[name]['GBps']:.0f} GB/s), "
            f"mean L_proj {res[name]['mean_L_proj']:.4g}, mean L_head {res[name]['mean_L_head']:.4g}")
    ckv_better = int((res["criticalkv"]["L_proj"] < res["h2o"]["L_proj"]).sum())
    mikv_better = int((res["mikv"]["L_proj"] < res["h2o"]["L_proj"]).sum())
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        h = 0
        sel = keep_ckv[h:h + 1].cpu().numpy()
        Kh, Vh = Kf[h:h + 1].cpu().numpy(), Vf[h:h + 1].cpu().numpy()
        Wh = W[h * d:(h + 1) * d].cpu().numpy()
        t1 = time.perf_counter()
        c1 = time.process_time()
        _, _, _, rLp = O.output_perturbation(qd[0, h:h + 1], Kh, Vh, Wh, keep=[sel[0]])
        el = time.perf_counter() - t1
        busy = (time.process_time() - c1) / el
        gpu_lp = float(res["criticalkv"]["L_proj"][h])
        cpu = {"value": el * H * 1e3, "unit": "ms per diagnostic (32 heads, extrapolated from 1)",
               "kind": "oracle", "cores": max(1, int(round(busy))), "cores_busy": busy,
               "sample": f"head 0 of {H}, CriticalKV kept set, fp64 numpy, {el:.2f} s",
               "parity": {"head": h, "L_proj_device": gpu_lp, "L_proj_oracle": float(rLp[0]),
                          "rel_diff": abs(gpu_lp - float(rLp[0])) / max(abs(float(rLp[0])), 1e-30)}}
    for r in res.values():
        r.pop("L_proj")
    best = min(res, key=lambda n: res[n]["us"])
    gbps = res[best]["GBps"]
    return {"metric": "output-perturbation diagnostic GB/s", "value": gbps, "unit": "GB/s",
            "higher_is_better": True, "steps": args.steps, "warmup": args.warmup, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": "perturbation_32k", "heads": H, "head_dim": d, "context": T + 1,
                       "hidden": hidden, "budget": B, "alpha": alpha, "low_bits": cfg.bits},
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS, "bytes_per_call": nbytes, "kernel_us": res[best]["us"],
                         "kernel": "mikv_output_perturbation (pert_attn_kernel streams K and V)"},
            "methods": res,
            "heads_criticalkv_below_h2o": ckv_better, "heads_mikv_below_h2o": mikv_better,
            "context": "the CriticalKV page reports lower perturbation in over 92% of Llama heads (real "
                       "weights); these are synthetic inputs",
            "cpu_baseline": cpu}


def bench_prefill(args, log):
    """Prefill-time kernels of the workload: the channel balancer (q and k
    max-abs scan, b) and the prefill build (top-H selection, FP16 rows and
    quantized low-bit rows), HBM-bound, GB/s from their algorithmic bytes;
    and the prompt heavy-hitter scores (causal attention column sums),
    MFMA-bound, TFLOP/s."""
    import torch
    from mixed_precision_decode_amd import _lib as L
    from mixed_precision_decode_amd import synth as S
    cfg = S.CONFIGS[args.workload]
    q, k, v, acc0 = S.prefill_tensors(cfg, args.seed)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    dims = L.Dims(batch=cfg.batch, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, group=cfg.G, bits=cfg.bits,
                  cap16=cfg.cap16, capq=cfg.T - cfg.B + 1)
    cache = L.Cache(dims)
    qg, kg, vg, ag = dev(q), dev(k), dev(v), dev(acc0)
    b = torch.empty((cfg.batch, cfg.hkv, cfg.d), dtype=torch.float32, device="cuda")
    ws_b = torch.empty(L.mikv_balance_workspace(dims, cfg.T), dtype=torch.uint8, device="cuda")
    ws_h = torch.empty(L.mikv_h2o_workspace(dims, cfg.T), dtype=torch.uint8, device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    fo = torch.empty((), dtype=torch.float32, device="cuda")
    n_u = cfg.batch * cfg.hkv
    bal_bytes = 2.0 * cfg.d * cfg.T * (cfg.batch * cfg.hq + n_u) + 4.0 * cfg.d * n_u
    build_bytes = n_u * (cfg.T * (4.0 * cfg.d + 4 + 4)          # k, v, acc0 read; slot map
                         + cfg.B * (4.0 * cfg.d + 8)             # FP16 rows + pos/acc written
                         + (cfg.T - cfg.B) * (2 * (cfg.d * cfg.bits / 8 + 4 * cfg.d / cfg.G) + 4))
    acc_s = torch.empty((cfg.batch, cfg.hkv, cfg.T), dtype=torch.float32, device="cuda")
    ws_s = torch.empty(L.mikv_prefill_scores_workspace(dims, cfg.T), dtype=torch.uint8, device="cuda")
    # prompt heavy-hitter scores: the causal score matrix of every query head,
    # T (T + 1) / 2 dot products of d, is the algorithmic work; the kernels
    # form it twice (softmax statistics, then column sums) in 32 x 32 tiles
    score_flops = 2.0 * cfg.d * cfg.T * (cfg.T + 1) / 2 * cfg.batch * cfg.hq
    nt = (cfg.T + 31) // 32
    exec_flops = 2 * 2.0 * cfg.d * 32 * 32 * nt * (nt + 1) / 2 * cfg.batch * cfg.hq
    res = {}
    for name, fn, nbytes in (
            ("balance", lambda: L.mikv_balance_prefill(dims, cfg.T, qg, kg, b, None, ws_b), bal_bytes),
            ("build", lambda: L.mikv_h2o_update_select(dims, cache, cfg.T, cfg.recent, cfg.H,
                                                       src=dict(k=kg, v=vg, acc0=ag, b=b), ws=ws_h), build_bytes),
            ("scores", lambda: L.mikv_prefill_scores(dims, cfg.T, qg, kg, acc_s, ws_s), None)):
        for _ in range(args.warmup):
            fn()
        evs = _events(args.steps)
        for e0, e1 in evs:
            torch.sum(flush, dim=0, out=fo)
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(e) for a, e in evs])) * 1e3
        if nbytes is None:
            tf = score_flops / (us * 1e-6) / 1e12
            res[name] = {"us": us, "algorithmic_flops": score_flops, "executed_flops": exec_flops,
                         "TFLOPs": tf, "executed_TFLOPs": exec_flops / (us * 1e-6) / 1e12,
                         "bound": "mfma", "peak_TFLOPs": 2500.0, "frac": tf / 2500.0}
            log(f"[bench] prefill {name} {us:.1f} us, {tf:.0f} TFLOP/s algorithmic, "
                f"{res[name]['executed_TFLOPs']:.0f} executed (fp16 MFMA)")
            continue
        res[name] = {"us": us, "bytes": nbytes, "GBps": nbytes / (us * 1e-6) / 1e9,
                     "frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        log(f"[bench] prefill {name} {us:.1f} us, {res[name]['GBps']:.0f} GB/s")
    return {"metric": "prefill balancer and build GB/s", "value": res["balance"]["GBps"], "unit": "GB/s",
            "higher_is_better": True, "steps": args.steps, "warmup": args.warmup, "dtype": "f32",
            "data": "synthetic", "config": {"workload": cfg.name}, "kernels": res}


def decode_run(cfg, args, log, K, W, KA, cpu_seconds):
    """Build the workload's cache on the device, then time it:
      - K decode steps (mikv_decode_step: attention + H2O update, two
        launches), HIP events at the step boundaries, after W warmup steps;
      - KA replays of one mikv_decode_attn call (split + merge) at a fixed
        length, events around the call: the call appends the same token and
        overwrites the same outputs each time, so replays leave the state as
        one call does;
      - KA replays of mikv_decode_attn_timed, whose events take the split
        kernel's own start and end (hipExtLaunchKernel);
    with an untimed read of 1 GiB before each timed launch. Then one more
    step runs untimed for the CPU baseline leg, which replays it on the
    oracle and compares. Returns the workload's entry of the JSON line."""
    import torch
    from mixed_precision_decode_amd import _lib as L
    from mixed_precision_decode_amd import synth as S
    total = W + K + 1
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    t0 = time.perf_counter()
    q, k, v, acc0 = S.prefill_tensors(cfg, args.seed)
    dims = L.Dims(batch=cfg.batch, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, group=cfg.G, bits=cfg.bits,
                  cap16=cfg.cap16, capq=cfg.scaled(steps=total).capq(), imp_bits=cfg.imp_bits,
                  key_tile=cfg.key_tile)
    cache = L.Cache(dims)
    b = torch.empty((cfg.batch, cfg.hkv, cfg.d), dtype=torch.float32, device="cuda")
    qg, kg = dev(q), dev(k)
    ws_b = torch.empty(L.mikv_balance_workspace(dims, cfg.T), dtype=torch.uint8, device="cuda")
    L.mikv_balance_prefill(dims, cfg.T, qg, kg, b, None, ws_b)
    del qg, q
    ws_h = torch.empty(L.mikv_h2o_workspace(dims, cfg.T), dtype=torch.uint8, device="cuda")
    L.mikv_h2o_update_select(dims, cache, cfg.T, cfg.recent, cfg.H,
                             src=dict(k=kg, v=dev(v), acc0=dev(acc0), b=b), ws=ws_h)
    torch.cuda.synchronize()
    del kg, ws_h, ws_b, k, v, acc0
    steps_np = [S.decode_tensors(cfg, args.seed, s) for s in range(total)]
    steps_in = [tuple(dev(x) for x in t) for t in steps_np]
    o = torch.empty((cfg.batch, cfg.hq, cfg.d), dtype=torch.float32, device="cuda")
    p16 = torch.empty((cfg.batch, cfg.hkv, cfg.cap16), dtype=torch.float32, device="cuda")
    ws = torch.zeros(L.mikv_decode_attn_workspace(dims, cfg.T + total), dtype=torch.uint8, device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")

    def do_flush(i):
        if args.flush == "read":
            torch.sum(flush, dim=0, out=flush_out)
        elif args.flush == "write":
            flush.fill_(float(i))
    log(f"[bench] {cfg.name}: cache built ({time.perf_counter() - t0:.1f}s); warmup {W}, timed {K}, "
        f"replays {KA}")

    def step_call(s, n_len):
        qd, kd, vd = steps_in[s]
        L.mikv_decode_step(dims, cache, n_len, cfg.recent, cfg.H, qd, kd, vd, b, o, p16, ws)

    graphs = {}
    if args.graph:
        # replay each timed step as one HIP graph, as a decode loop could
        for s in range(W, W + K):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_call(s, cfg.T + s + 1)
            graphs[s] = g
        torch.cuda.synchronize()
    N = cfg.T
    for s in range(W):
        N += 1
        do_flush(s)
        step_call(s, N)
    torch.cuda.synchronize()
    Ev = lambda: torch.cuda.Event(enable_timing=True)
    evs = [(Ev(), Ev()) for _ in range(K)]
    lens = []
    tw0 = time.perf_counter()
    for i in range(K):
        N += 1
        do_flush(i)
        evs[i][0].record()
        if W + i in graphs:
            graphs[W + i].replay()
        else:
            step_call(W + i, N)
        evs[i][1].record()
        lens.append(N)
    torch.cuda.synchronize()
    wall = time.perf_counter() - tw0
    # replays of the next step's attention call at length N + 1
    s_next = W + K
    qd, kd, vd = steps_in[s_next]
    eva = [(Ev(), Ev()) for _ in range(KA)]
    for i in range(KA):
        do_flush(i)
        eva[i][0].record()
        L.mikv_decode_attn(dims, cache, N + 1, qd, kd, vd, b, o, p16, ws)
        eva[i][1].record()
    evk = [(Ev(), Ev()) for _ in range(KA)]
    for i in range(KA):
        do_flush(i)
        L.mikv_decode_attn_timed(dims, cache, N + 1, qd, kd, vd, b, o, p16, ws, *evk[i])
    torch.cuda.synchronize()
    step_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    attn_ms = np.array([e[0].elapsed_time(e[1]) for e in eva])
    split_ms = np.array([e[0].elapsed_time(e[1]) for e in evk])
    lens = np.array(lens)
    ms_per_step = float(step_ms.mean())
    value = float(cfg.batch * lens.mean() / (ms_per_step * 1e-3))
    kbytes = float(split_bytes(cfg, N + 1))
    abytes = float(attn_bytes(cfg, N + 1))
    split_us = float(np.median(split_ms)) * 1e3
    call_us = float(np.median(attn_ms)) * 1e3
    k_gbps = kbytes / (split_us * 1e-6) / 1e9
    a_gbps = abytes / (call_us * 1e-6) / 1e9
    sbytes = np.array([attn_bytes(cfg, n) + h2o_bytes(cfg) for n in lens], dtype=np.float64)
    s_gbps = float((sbytes / (step_ms * 1e-3)).mean() / 1e9)
    log(f"[bench] {cfg.name}: split kernel {split_us:.1f} us median ({k_gbps:.0f} GB/s, "
        f"{k_gbps / HBM_PEAK_GBPS:.3f}), attn call {call_us:.1f} us median ({a_gbps:.0f} GB/s, "
        f"{a_gbps / HBM_PEAK_GBPS:.3f}), step {ms_per_step * 1e3:.1f} us mean "
        f"({np.median(step_ms) * 1e3:.1f} median), {value:.3g} KV-tokens/s")
    cpu = None
    if cpu_seconds > 0:
        # one more decode step, untimed: the oracle replays it from the same
        # state (sequence 0) and compares
        before = {kk: getattr(cache, kk)[:1].cpu().numpy() for kk in cache.names}
        before["group"], before["bits"], before["imp_bits"] = cfg.G, cfg.bits, cache.imp_bits
        before["key_tile"] = cache.key_tile
        N += 1
        step_call(s_next, N)
        after = {kk: getattr(cache, kk)[:1].cpu().numpy() for kk in cache.names}
        gpu = {"o": o[:1].cpu().numpy(), "after": after}
        qn, kn, vn = (x[:1] for x in steps_np[s_next])
        cpu = cpu_baseline(cfg, before, b[:1].cpu().numpy(), N, qn, kn, vn, gpu, cpu_seconds)
        log(f"[bench] {cfg.name}: cpu oracle {cpu['value']:.3g} KV-tokens/s ({cpu['sample']}); "
            f"parity {cpu['parity']}")
    del cache, steps_in, ws, flush
    torch.cuda.empty_cache()
    traffic_ok = not args.set
    return {
        "workload": cfg.name, "value": value, "unit": "KV-tokens/s", "ms_per_step": ms_per_step,
        "ms_per_step_median": float(np.median(step_ms)), "steps": K, "warmup": W,
        "config": {"workload": cfg.name, "batch": cfg.batch, "q_heads": cfg.hq, "kv_heads": cfg.hkv,
                   "head_dim": cfg.d, "context": cfg.T, "low_bits": cfg.bits,
                   "importance_bits": cfg.imp_bits, "key_tile": cfg.key_tile,
                   "important_pct": cfg.pct, "recent": cfg.recent, "group": cfg.G,
                   "cache_flush_per_step": args.flush,
                   "step_launch": "hip_graph" if args.graph else "eager"},
        "roofline": {"bound": "hbm", "achieved": k_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": k_gbps / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic(cfg.name) if traffic_ok else None,
                     "launches_timed": KA, "statistic": "median", "kernel": split_kernel_name(cfg),
                     "kernel_us": split_us, "bytes_per_launch": kbytes,
                     "timing": "hipExtLaunchKernel start/stop events of the kernel itself"},
        "attn_call": {"kernels": f"{split_kernel_name(cfg)} + decode_merge_kernel (one mikv_decode_attn call)",
                      "us": call_us, "bytes": abytes, "GBps": a_gbps, "frac": a_gbps / HBM_PEAK_GBPS,
                      "launches_timed": KA, "statistic": "median",
                      "traffic": recorded_traffic(cfg.name, "call_traffic_bytes") if traffic_ok else None,
                      "timing": "HIP events recorded on the stream before and after the call"},
        "step_hbm_gbps": s_gbps,
        "wall_ms_per_step_incl_flush": wall / K * 1e3,
        "cpu_baseline": cpu,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--attn-steps", type=int, default=60,
                    help="replays of the attention call, and as many of the split kernel with its "
                         "own start/stop events (medians reported)")
    ap.add_argument("--workload", default="llama2_7b_layer")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only --workload (by default the other decode workloads follow it in "
                         "the same run, under \"configs\")")
    ap.add_argument("--seed", type=int, default=1001)
    ap.add_argument("--set", action="append", default=[], metavar="FIELD=INT",
                    help="override an integer field of the workload (e.g. pct=100)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--extra-cpu-seconds", type=float, default=4.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", choices=("read", "write", "none"), default="read")
    ap.add_argument("--graph", type=int, default=0,
                    help="1: replay each timed step as one HIP graph; 0 (default): eager "
                         "launches, measured faster on MI355X for this step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference kernel for HBM counters)")
    ap.add_argument("--criticalkv", action="store_true",
                    help="only time the CriticalKV prefill select (32 heads, 32K tokens); one JSON line")
    ap.add_argument("--quantize", action="store_true",
                    help="only time mikv_quantize_tokens on the workload's prompt rows; one JSON line")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only time a plain streaming read of one split-kernel launch's bytes; one JSON line")
    ap.add_argument("--perturbation", action="store_true",
                    help="only time the output-perturbation diagnostic of H2O, CriticalKV and MiKV "
                         "(32 heads x 32K tokens); one JSON line")
    ap.add_argument("--prefill", action="store_true",
                    help="only time the workload's prefill kernels (balancer, build, heavy-hitter "
                         "scores); one JSON line")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.criticalkv or args.prefill or args.read_ceiling or args.quantize or args.perturbation:
        log = lambda *a: print(*a, file=sys.stderr, flush=True)
        fn = (bench_criticalkv if args.criticalkv else bench_prefill if args.prefill
              else bench_quantize if args.quantize else bench_perturbation if args.perturbation
              else read_ceiling)
        print(json.dumps(fn(args, log)), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the MiKV path runs on one GPU only; --gpus must be 1 "
              "(every (sequence, kv head) unit is independent, so the path would shard by unit "
              "with no exchange; no multi-GPU figure is measured here)",
              file=sys.stderr)
        sys.exit(2)

    from mixed_precision_decode_amd import synth as S

    cfg = S.CONFIGS[args.workload]
    if args.set:
        cfg = cfg.scaled(**{kv.split("=")[0]: int(kv.split("=")[1]) for kv in args.set})
    K, W, KA = args.steps, args.warmup, args.attn_steps
    if W + K + 1 > cfg.steps:
        ap.error(f"workload {cfg.name} defines {cfg.steps} decode steps: --warmup + --steps + 1 "
                 f"must not exceed it (got {W + K + 1})")
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    head = decode_run(cfg, args, log, K, W, KA, cpu_s)
    extra = []
    if not args.no_extra and not args.set:
        for name in ("llama3_8b_32k", "gqa_throughput", "llama2_7b_imp4", "llama2_7b_kchan"):
            if name == cfg.name:
                continue
            c2 = S.CONFIGS[name]
            w2 = min(W, c2.steps - 2)
            k2 = min(K, c2.steps - w2 - 1)
            extra.append(decode_run(c2, args, log, k2, w2, KA,
                                    0.0 if args.no_cpu_baseline else args.extra_cpu_seconds))
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "attn_call": head["attn_call"],
        "ms_per_step_median": head["ms_per_step_median"],
        "step_hbm_gbps": head["step_hbm_gbps"],
        "wall_ms_per_step_incl_flush": head["wall_ms_per_step_incl_flush"],
        "parity": None if head["cpu_baseline"] is None else head["cpu_baseline"]["parity"],
        "cpu_baseline": head["cpu_baseline"],
        "configs": [{kk: e[kk] for kk in ("workload", "value", "unit", "ms_per_step", "ms_per_step_median",
                                           "steps", "warmup", "config", "roofline", "attn_call",
                                           "cpu_baseline")}
                    for e in extra],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
