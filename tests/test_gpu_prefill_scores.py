"""Parity of the prompt heavy-hitter scores (mikv_prefill_scores, HIP on
matrix cores) with the CPU oracle's causal-attention column sums.

Tolerance (fp32 scores and sums vs the fp64 oracle): max|gpu - oracle| <=
2e-3 * max|oracle| per tensor. At full sizes, where the oracle's T x T
matrices are too large for some shapes, sampled (sequence, kv head) units are
compared and every unit is checked for conservation: each causal softmax row
sums to 1, so a unit's scores sum to (hq/hkv) * T.
"""
import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_decode_amd import _lib as L
from mixed_precision_decode_amd import synth as S

pytestmark = pytest.mark.gpu
F64 = np.float64
TOL = 2e-3


def _gpu_scores(cfg, q, k):
    dims = L.Dims(batch=cfg.batch, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, group=cfg.G, bits=cfg.bits,
                  cap16=cfg.cap16, capq=cfg.capq())
    acc = torch.full((cfg.batch, cfg.hkv, cfg.T), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(L.mikv_prefill_scores_workspace(dims, cfg.T), dtype=torch.uint8, device="cuda")
    qd = torch.from_numpy(np.ascontiguousarray(q)).cuda()
    kd = torch.from_numpy(np.ascontiguousarray(k)).cuda()
    L.mikv_prefill_scores(dims, cfg.T, qd, kd, acc, ws)
    torch.cuda.synchronize()
    return acc.cpu().numpy()


def _close(gpu, ref, what):
    err = np.max(np.abs(gpu.astype(F64) - ref))
    scale = np.max(np.abs(ref))
    assert err <= TOL * scale, f"{what}: max err {err:.3e} > {TOL} * {scale:.3e}"


def _conserved(acc, cfg):
    sums = acc.astype(F64).sum(-1)
    want = cfg.rep * cfg.T
    assert np.all(np.isfinite(acc)) and np.all(acc >= 0)
    assert np.max(np.abs(sums - want)) <= 1e-4 * want, (sums.min(), sums.max(), want)


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),                                            # d 64, one head, T 256
    ("tiny", dict(T=1)),
    ("tiny", dict(T=31, hq=4, hkv=2)),
    ("tiny", dict(T=33, hq=4, hkv=1)),
    ("tiny", dict(T=300, hq=8, hkv=2, batch=2)),             # ragged, several 128-row blocks
    ("tiny", dict(T=129, hq=4, hkv=1, d=128)),
    ("llama3_8b_32k", dict(T=1000, hq=8, hkv=2)),
    ("gqa_throughput", dict(batch=2, T=517)),
    ("llama2_7b_layer", dict(batch=1, hq=2, hkv=2, T=640)),
])
def test_prefill_scores_parity(name, over):
    cfg = S.CONFIGS[name].scaled(**over)
    print(f"prefill_scores {name} {over}", flush=True)
    q, k, _, _ = S.prefill_tensors(cfg, 7)
    acc = _gpu_scores(cfg, q, k)
    ref = O.prefill_scores(q, k)
    _close(acc, ref, "acc0")
    _conserved(acc, cfg)


@pytest.mark.parametrize("name", ["llama2_7b_layer", "gqa_throughput", "llama3_8b_32k"])
def test_prefill_scores_full_size(name):
    """The workloads' full prompts: every unit conserves its mass; sampled
    units whose T x T matrices the oracle holds match it."""
    cfg = S.CONFIGS[name]
    print(f"prefill_scores full size {name}", flush=True)
    q, k, _, _ = S.prefill_tensors(cfg, 1000 + list(S.CONFIGS).index(name))
    acc = _gpu_scores(cfg, q, k)
    _conserved(acc, cfg)
    if cfg.T <= 4096:
        rep = cfg.rep
        for n, g in ((0, 0), (cfg.batch - 1, cfg.hkv - 1)):
            ref = O.prefill_scores(q[n:n + 1, g * rep:(g + 1) * rep], k[n:n + 1, g:g + 1])
            _close(acc[n, g], ref[0, 0], f"acc0 unit ({n}, {g})")
