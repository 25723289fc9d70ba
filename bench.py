"""Benchmark of the MiKV mixed-precision decode path on one MI355X.

A step is one decode step of the whole batch (mikv_decode_step):
mixed-precision attention over both cache tiers (append + scores + softmax +
value sum) and the H2O accumulate / re-select / demote, in two launches (the
attention's merge kernel also runs the H2O update). The cache is built once
before timing (balancer + prefill build on the GPU) from seeded synthetic
inputs; every step consumes a new seeded (q, k, v) token per sequence and
kv head, so the low-bit tier grows by one token per step.

Before each timed step an untimed read of a 1 GiB device buffer evicts the
caches (MI355X has a 256 MB Infinity Cache, larger than the per-step working
set of the configs), so each step streams its cache from HBM. The flush
reads rather than writes: a written flush leaves the Infinity Cache full of
dirty lines whose write-back would then compete with the measured kernel
(--flush write shows that case, --flush none the warm-cache case). Step and
kernel times come from HIP events recorded on the stream the kernels run on.

The JSON line's roofline is the dominant kernel's: the split kernel, timed
by start/stop events of its own launch (mikv_decode_attn_timed); the call
(split + merge) is reported beside it. Other modes, one JSON line each:
--prefill (balancer, prefill build, prompt heavy-hitter scores), --quantize
(mikv_quantize_tokens on every prompt row), --criticalkv (the CriticalKV
select, 32 heads x 32K tokens), --read-ceiling (a plain streaming read of
one split launch's bytes), --calibrate-copy (the 1 GiB copy that scales the
HBM counters).

Prints one JSON line (rank 0). --gpus N > 1 is refused: the path runs on one
GPU.
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


def attn_bytes(cfg, N):
    """Algorithmic bytes of one decode-attention launch at length N (new
    token included): FP16 tier rows read (cap16-1) plus the new row read and
    appended, low-bit rows (codes + fp16 scale/zero per group, K and V), q, b,
    o and p16."""
    d, G = cfg.d, cfg.G
    nq = N - cfg.cap16
    per_unit = ((cfg.cap16 - 1) * 4 * d + 4 * d + 4 * d
                + nq * 2 * (d * cfg.bits // 8 + 4 * (d // G))
                + cfg.rep * d * 2 + d * 4 + cfg.rep * d * 4 + cfg.cap16 * 4)
    return per_unit * cfg.batch * cfg.hkv


def split_bytes(cfg, N):
    """Algorithmic bytes of one split-kernel launch at length N: everything
    attn_bytes counts except o and p16, which the merge kernel writes."""
    return attn_bytes(cfg, N) - (cfg.rep * cfg.d * 4 + cfg.cap16 * 4) * cfg.batch * cfg.hkv


def h2o_bytes(cfg):
    """acc16 read+write, p16 and pos16 read per FP16 slot; the demoted K/V
    rows read and written as codes."""
    d = cfg.d
    per_unit = cfg.cap16 * 16 + 4 * d + 2 * (d * cfg.bits // 8 + 4 * (d // cfg.G)) + 16
    return per_unit * cfg.batch * cfg.hkv


def cpu_baseline(cfg, cache_np, b_np, N, seed, step, budget_s):
    """The CPU oracle (as it stands) on a bounded sample of the same workload:
    one sequence's decode step (all its kv heads), repeated until budget_s."""
    import oracle as O
    from mixed_precision_decode_amd import synth as S
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    sub = {k: (v[:1].copy() if isinstance(v, np.ndarray) else v) for k, v in cache_np.items()}
    qd, kd, vd = S.decode_tensors(cfg.scaled(batch=1), seed, step)
    reps = 0
    t0 = time.perf_counter()
    c0 = time.process_time()
    while True:
        O.decode_step(sub, N, qd, kd, vd, b_np[:1], cfg.recent, cfg.H)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    # cores actually used: the process's CPU time over the wall time (numpy's
    # elementwise work is single-threaded; only its BLAS calls use the pool)
    busy = (time.process_time() - c0) / el
    return {"value": reps * N / el, "unit": "KV-tokens/s", "cores": max(1, int(round(busy))),
            "cores_busy": busy, "blas_threads": int(threads), "kind": "oracle",
            "sample": (f"{reps} oracle decode steps of 1 of {cfg.batch} sequences "
                       f"({cfg.hkv} kv heads, N={N}), fp64 numpy, {el:.1f} s; "
                       f"host os.cpu_count()={os.cpu_count()}")}


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
    us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
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
        us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
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
    b1 = int(np.floor(np.float64(np.float32(cfg.alpha)) * budget))
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
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
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
        us = float(np.mean([a.elapsed_time(e) for a, e in evs])) * 1e3
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--attn-steps", type=int, default=20,
                    help="decode steps timed around the attention call alone, and as many "
                         "timed at the split kernel's own start and end")
    ap.add_argument("--workload", default="llama2_7b_layer")
    ap.add_argument("--seed", type=int, default=1001)
    ap.add_argument("--set", action="append", default=[], metavar="FIELD=INT",
                    help="override an integer field of the workload (e.g. pct=100)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
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
    ap.add_argument("--prefill", action="store_true",
                    help="only time the workload's prefill kernels (balancer, build, heavy-hitter "
                         "scores); one JSON line")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.criticalkv or args.prefill or args.read_ceiling or args.quantize:
        log = lambda *a: print(*a, file=sys.stderr, flush=True)
        fn = (bench_criticalkv if args.criticalkv else bench_prefill if args.prefill
              else bench_quantize if args.quantize else read_ceiling)
        print(json.dumps(fn(args, log)), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the MiKV path runs on one GPU only; --gpus must be 1 "
              "(the path shards by (sequence, kv head) with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from mixed_precision_decode_amd import _lib as L
    from mixed_precision_decode_amd import synth as S

    cfg = S.CONFIGS[args.workload]
    if args.set:
        cfg = cfg.scaled(**{kv.split("=")[0]: int(kv.split("=")[1]) for kv in args.set})
    K, W, KA = args.steps, args.warmup, args.attn_steps
    total = K + W + 2 * KA
    if total > cfg.steps:
        ap.error(f"workload {cfg.name} defines {cfg.steps} decode steps: --warmup + --steps + "
                 f"2 * --attn-steps must not exceed it (got {total})")
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    log = lambda *a: print(*a, file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    q, k, v, acc0 = S.prefill_tensors(cfg, args.seed)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f}s")
    dims = L.Dims(batch=cfg.batch, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, group=cfg.G, bits=cfg.bits,
                  cap16=cfg.cap16, capq=cfg.T - cfg.B + total)
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
    del kg, ws_h, ws_b
    steps_in = [tuple(dev(x) for x in S.decode_tensors(cfg, args.seed, s)) for s in range(total)]
    o = torch.empty((cfg.batch, cfg.hq, cfg.d), dtype=torch.float32, device="cuda")
    p16 = torch.empty((cfg.batch, cfg.hkv, cfg.cap16), dtype=torch.float32, device="cuda")
    ws = torch.zeros(L.mikv_decode_attn_workspace(dims, cfg.T + total), dtype=torch.uint8,
                     device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")

    def do_flush(i):
        if args.flush == "read":
            torch.sum(flush, dim=0, out=flush_out)
        elif args.flush == "write":
            flush.fill_(float(i))
    log(f"[bench] cache built ({time.perf_counter() - t0:.1f}s); warmup {W}, timed {K}")

    N = cfg.T
    cpu_state = None

    def attn_call(s, n_len, split_ev=None):
        qd, kd, vd = steps_in[s]
        if split_ev is None:
            L.mikv_decode_attn(dims, cache, n_len, qd, kd, vd, b, o, p16, ws)
        else:
            # the events take the split kernel's own start and end
            L.mikv_decode_attn_timed(dims, cache, n_len, qd, kd, vd, b, o, p16, ws, *split_ev)

    def step_call(s, n_len):
        qd, kd, vd = steps_in[s]
        L.mikv_decode_step(dims, cache, n_len, cfg.recent, cfg.H, qd, kd, vd, b, o, p16, ws)

    def h2o_call(n_len):
        L.mikv_h2o_update_select(dims, cache, n_len, cfg.recent, cfg.H, p16=p16)

    # Optionally replay each timed step (decode attention + H2O) as one HIP
    # graph, as a decode loop could.
    graphs = {}
    if args.graph:
        for s in range(W, W + K):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_call(s, cfg.T + s + 1)
            graphs[s] = g
        torch.cuda.synchronize()

    def one_step(s, ev_start=None, ev_attn=None, ev_end=None, split_ev=None):
        nonlocal N
        N += 1
        assert N == cfg.T + s + 1
        if ev_start is not None:
            ev_start.record()
        if ev_attn is None:
            # one decode step: mikv_decode_step (attention + H2O, two launches)
            if s in graphs:
                graphs[s].replay()
            else:
                step_call(s, N)
        else:
            # attention-only timing: mikv_decode_attn, then the H2O call
            attn_call(s, N, split_ev)
            if ev_attn is not None:
                ev_attn.record()
            h2o_call(N)
        if ev_end is not None:
            ev_end.record()

    for s in range(W):
        do_flush(s)
        one_step(s)
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        cpu_state = (cache.to_numpy(), b.cpu().numpy(), N + 1, W)
    # timed steps: events only at the step boundaries (an event between two
    # kernels costs a few microseconds of its own)
    Ev = lambda: torch.cuda.Event(enable_timing=True)
    evs = [(Ev(), Ev()) for _ in range(K)]
    lens = []
    torch.cuda.synchronize()
    tw0 = time.perf_counter()
    for i in range(K):
        do_flush(i)
        one_step(W + i, ev_start=evs[i][0], ev_end=evs[i][1])
        lens.append(N)
    torch.cuda.synchronize()
    wall = time.perf_counter() - tw0
    # attention alone, two passes of KA decode steps each:
    #  - events on the stream around each mikv_decode_attn call (split + merge);
    #  - mikv_decode_attn_timed, whose events take the start and end of the
    #    split kernel itself, the dominant kernel (hipExtLaunchKernel; such a
    #    launch leaves a gap of a few microseconds before the next kernel, so
    #    these calls are not the ones the call-level time comes from)
    eva = [(Ev(), Ev()) for _ in range(KA)]
    alens = []
    for i in range(KA):
        do_flush(i)
        one_step(W + K + i, ev_start=eva[i][0], ev_attn=eva[i][1])
        alens.append(N)
    evk = [(Ev(), Ev()) for _ in range(KA)]
    klens = []
    for i in range(KA):
        do_flush(i)
        one_step(W + K + KA + i, ev_attn=Ev(), split_ev=evk[i])
        klens.append(N)
    torch.cuda.synchronize()
    step_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    attn_ms = np.array([e[0].elapsed_time(e[1]) for e in eva])
    split_ms = np.array([e[0].elapsed_time(e[1]) for e in evk])
    lens = np.array(lens)
    ms_per_step = float(step_ms.mean())
    value = float(cfg.batch * lens.mean() / (ms_per_step * 1e-3))
    abytes = np.array([attn_bytes(cfg, n) for n in alens], dtype=np.float64)
    a_gbps = float((abytes / (attn_ms * 1e-3)).mean() / 1e9)
    kbytes = np.array([split_bytes(cfg, n) for n in klens], dtype=np.float64)
    k_gbps = float(kbytes.mean() / (split_ms.mean() * 1e-3) / 1e9)
    sbytes = np.array([attn_bytes(cfg, n) + h2o_bytes(cfg) for n in lens], dtype=np.float64)
    s_gbps = float((sbytes / (step_ms * 1e-3)).mean() / 1e9)
    log(f"[bench] split kernel {split_ms.mean() * 1e3:.1f} us ({k_gbps:.0f} GB/s), attn call "
        f"{attn_ms.mean() * 1e3:.1f} us ({a_gbps:.0f} GB/s), step "
        f"{ms_per_step * 1e3:.1f} us ({s_gbps:.0f} GB/s), wall incl. flush {wall / K * 1e3:.3f} ms/step")

    cpu = None
    if cpu_state is not None:
        cache_np, b_np, Nc, st = cpu_state
        cpu = cpu_baseline(cfg, cache_np, b_np, Nc, args.seed, st, args.cpu_seconds)
        log(f"[bench] cpu oracle {cpu['value']:.3g} KV-tokens/s ({cpu['sample']})")

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "q_heads": cfg.hq, "kv_heads": cfg.hkv,
                   "head_dim": cfg.d, "context": cfg.T, "low_bits": cfg.bits,
                   "important_pct": cfg.pct, "recent": cfg.recent, "group": cfg.G,
                   "cache_flush_per_step": args.flush, "step_launch": "hip_graph" if args.graph else "eager"},
        "roofline": {"bound": "hbm", "achieved": k_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": k_gbps / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic(cfg.name) if not args.set else None,
                     "launches_timed": KA, "kernel": "decode_split_kernel",
                     "kernel_us": float(split_ms.mean() * 1e3),
                     "bytes_per_launch": float(kbytes.mean()),
                     "timing": "hipExtLaunchKernel start/stop events of the kernel itself"},
        "attn_call": {"kernels": "decode_split_kernel + decode_merge_kernel (one mikv_decode_attn call)",
                      "us": float(attn_ms.mean() * 1e3), "bytes": float(abytes.mean()),
                      "GBps": a_gbps, "frac": a_gbps / HBM_PEAK_GBPS,
                      "traffic": recorded_traffic(cfg.name, "call_traffic_bytes") if not args.set else None,
                      "timing": "HIP events recorded on the stream before and after the call"},
        "step_hbm_gbps": s_gbps,
        "wall_ms_per_step_incl_flush": wall / K * 1e3,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
