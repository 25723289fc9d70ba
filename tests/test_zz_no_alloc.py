"""mikv_decode_step_noalloc (fixed device scratch, no allocation) against
mikv_decode_step with a caller workspace: bit-identical outputs and caches,
on two calls in a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

from mixed_precision_decode_amd import _lib as L
from mixed_precision_decode_amd import synth as S

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _prefilled(cfg, seed):
    q, k, v, acc0 = S.prefill_tensors(cfg, seed)
    dims = L.Dims(batch=cfg.batch, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, group=cfg.G, bits=cfg.bits,
                  cap16=cfg.cap16, capq=cfg.capq())
    cache = L.Cache(dims)
    b = torch.empty((cfg.batch, cfg.hkv, cfg.d), dtype=torch.float32, device="cuda")
    ws_b = torch.empty(max(1, L.mikv_balance_workspace(dims, cfg.T)), dtype=torch.uint8, device="cuda")
    L.mikv_balance_prefill(dims, cfg.T, _dev(q), _dev(k), b, None, ws_b)
    ws_h = torch.empty(max(1, L.mikv_h2o_workspace(dims, cfg.T)), dtype=torch.uint8, device="cuda")
    L.mikv_h2o_update_select(dims, cache, cfg.T, cfg.recent, cfg.H,
                             src=dict(k=_dev(k), v=_dev(v), acc0=_dev(acc0), b=b), ws=ws_h)
    return dims, cache, b


def _outputs(cfg, dims):
    return (torch.full((cfg.batch, cfg.hq, cfg.d), 7.0, dtype=torch.float32, device="cuda"),
            torch.full((cfg.batch, cfg.hkv, cfg.cap16), 7.0, dtype=torch.float32, device="cuda"),
            torch.full((cfg.batch, cfg.hkv), -5, dtype=torch.int32, device="cuda"))


def _same(a, b):
    a, b = a.cpu().numpy(), b.cpu().numpy()
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_noalloc_matches_workspace_entry_two_calls():
    # first call: 4 x 8 GQA units of 4 heads at T 900 (two splits per unit);
    # second, smaller: 1 x 2 units at T 256 (single-head tiles, more splits)
    cfgs = [S.CONFIGS["gqa_throughput"].scaled(batch=4, T=900),
            S.CONFIGS["tiny"].scaled(hq=4, hkv=2)]
    runs = []
    for i, cfg in enumerate(cfgs):
        dims_w, cache_w, b_w = _prefilled(cfg, 50 + i)
        dims_n, cache_n, b_n = _prefilled(cfg, 50 + i)
        qd, kd, vd = (_dev(x) for x in S.decode_tensors(cfg, 50 + i, 0))
        ws = torch.empty(L.mikv_decode_attn_workspace(dims_w, cfg.T + 1), dtype=torch.uint8, device="cuda")
        assert ws.numel() <= L.mikv_decode_step_noalloc_limit()
        runs.append((cfg, dims_w, cache_w, b_w, dims_n, cache_n, b_n, (qd, kd, vd), ws,
                     _outputs(cfg, dims_w), _outputs(cfg, dims_n)))
    torch.cuda.synchronize()
    # the two fixed-scratch calls back to back, larger input first
    for cfg, _, _, _, dims_n, cache_n, b_n, (qd, kd, vd), _, _, (o, p16, dpos) in runs:
        print(f"noalloc decode step: batch {cfg.batch}, {cfg.hq}/{cfg.hkv} heads, T {cfg.T}", flush=True)
        L.mikv_decode_step_noalloc(dims_n, cache_n, cfg.T + 1, cfg.recent, cfg.H, qd, kd, vd, b_n, o, p16,
                                   demoted_pos=dpos)
    for cfg, dims_w, cache_w, b_w, _, _, _, (qd, kd, vd), ws, (o, p16, dpos), _ in runs:
        L.mikv_decode_step(dims_w, cache_w, cfg.T + 1, cfg.recent, cfg.H, qd, kd, vd, b_w, o, p16, ws,
                           demoted_pos=dpos)
    torch.cuda.synchronize()
    for cfg, _, cache_w, _, _, cache_n, _, _, _, out_w, out_n in runs:
        for a, b in zip(out_w, out_n):
            assert _same(a, b), cfg
        for key in L.Cache.NAMES:
            assert _same(getattr(cache_w, key), getattr(cache_n, key)), (cfg, key)
        assert int(out_n[2].min()) >= 0   # every unit demoted a token


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """A shape whose partial results exceed the fixed scratch is refused
    with MIKV_ERR_SCRATCH before anything is enqueued."""
    cfg = S.CONFIGS["tiny"].scaled(batch=4096, hq=32, hkv=32, T=40, pct=50, recent=4)
    dims = L.Dims(batch=cfg.batch, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, group=cfg.G, bits=cfg.bits,
                  cap16=cfg.cap16, capq=cfg.capq())
    assert L.mikv_decode_attn_workspace(dims, cfg.T + 1) > L.mikv_decode_step_noalloc_limit()
    cache = L.Cache(dims)
    o, p16, dpos = _outputs(cfg, dims)
    z = torch.zeros((cfg.batch, cfg.hq, cfg.d), dtype=torch.float16, device="cuda")
    zk = torch.zeros((cfg.batch, cfg.hkv, cfg.d), dtype=torch.float16, device="cuda")
    b = torch.ones((cfg.batch, cfg.hkv, cfg.d), dtype=torch.float32, device="cuda")
    with pytest.raises(L.MikvError) as e:
        L.mikv_decode_step_noalloc(dims, cache, cfg.T + 1, cfg.recent, cfg.H, z, zk, zk, b, o, p16)
    assert e.value.status == L.MIKV_ERR_SCRATCH
