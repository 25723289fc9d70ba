"""Seeded synthetic workloads for the mixed-precision KV-cache path.

This module only draws random numbers and names workload shapes. It holds
none of the method's arithmetic: no balancer, no quantizer, no attention, no
selection. Both the HIP path (through the binding) and the CPU oracle consume
the arrays it returns.

Workloads stand in for the shapes the pages evaluate on (no dataset or model
weight is used):
  * a Llama-2-7B-shaped attention layer (32 MHA heads of 128 channels) at the
    batch 8 x 4096-token setting of the memory-footprint analysis on the
    arXiv 2402.18096 summary page (section 4.4);
  * a Llama-3-8B-shaped GQA layer (32 query / 8 kv heads) at 32K context;
  * a GQA throughput batch;
  * the CriticalKV 32K-context, batch-1 setting (gist.science summary of
    arXiv 2502.03805, experiments / efficiency);
  * the reduced-precision importance cache of Table 3 on the velog notes
    page (20% importance at INT4 or INT8, 2-bit retention), on the
    Llama-2-7B layer shape.

Value model. q, k, v are N(0,1) draws cast to fp16 with round-to-nearest-even.
Query/key outliers follow the observations on the velog notes page
("Key contributions 2) Outlier-aware"): outlier channels sit at fixed
positions along the sequence and appear duplicated after RoPE, so each kv
head gets ``pairs`` channel pairs {c, c + d/2}; the N(0,1) samples on those
channels of q and k are multiplied by ``factor``. The same channels are used
for every query head that shares the kv head.

The prefill heavy-hitter scores ``acc0`` (accumulated attention of the prompt)
are a seeded stand-in: log-normal draws scaled so that the total mass equals
``rep * T`` (every prefill query row of every query head in the group carries
probability mass 1), rounded to a 2^-10 grid so that exact ties occur, with
about 5% exact zeros. The pages do not describe how H2O initialises its scores,
so for the decode workloads this input is drawn, with exact ties on purpose;
the library's mikv_prefill_scores computes acc0 from a prompt's q and k.

Every array of one (sequence, kv head) unit comes from its own generator
seeded by ``(seed, stream, n, g[, step])`` so that any unit can be drawn on
its own, and full tensors are the stack of their units.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "DecodeConfig", "CriticalKVConfig", "CONFIGS", "CKV_CONFIGS",
    "outlier_channels", "unit_prefill", "unit_acc0", "unit_decode",
    "prefill_tensors", "decode_tensors", "criticalkv_inputs",
]


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    hq: int
    hkv: int
    d: int
    T: int
    bits: int
    pct: int          # important (FP16) share of the prompt, in percent
    recent: int       # recent-window length R (inside the FP16 budget)
    steps: int        # decode steps of the workload
    pairs: int        # outlier channel pairs per kv head
    factor: float     # outlier magnitude multiplier
    group: int = 0    # channels per quantization group (0: d/2)
    imp_bits: int = 16  # importance tier: 16 = fp16 rows, 8 or 4 = codes
    key_tile: int = 0   # 0: per-token keys; 64: per-channel key tiles + token buffer

    @property
    def rep(self) -> int:
        return self.hq // self.hkv

    @property
    def G(self) -> int:
        return self.group if self.group else self.d // 2

    @property
    def B(self) -> int:
        """Important-set size floor(pct/100 * T), fixed after prefill."""
        return (self.T * self.pct) // 100

    @property
    def H(self) -> int:
        return self.B - self.recent

    @property
    def cap16(self) -> int:
        return self.B + 1

    def capq(self, steps: int | None = None) -> int:
        s = self.steps if steps is None else steps
        c = self.T - self.B + s
        if self.key_tile:  # whole tiles
            c = -(-c // self.key_tile) * self.key_tile
        return c

    def scaled(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class CriticalKVConfig:
    name: str
    H: int
    d: int
    hidden: int
    T: int
    pct: int          # budget as percent of T
    alpha: float
    sigma: float      # std of the fp16 attention logits

    @property
    def budget(self) -> int:
        return (self.T * self.pct) // 100


CONFIGS = {
    "tiny": DecodeConfig("tiny", batch=1, hq=1, hkv=1, d=64, T=256, bits=4, pct=20,
                         recent=16, steps=32, pairs=1, factor=15.0),
    "llama2_7b_layer": DecodeConfig("llama2_7b_layer", batch=8, hq=32, hkv=32, d=128, T=4096,
                                    bits=4, pct=20, recent=64, steps=128, pairs=2, factor=20.0),
    "llama3_8b_32k": DecodeConfig("llama3_8b_32k", batch=1, hq=32, hkv=8, d=128, T=32768,
                                  bits=2, pct=10, recent=64, steps=64, pairs=2, factor=20.0),
    "gqa_throughput": DecodeConfig("gqa_throughput", batch=64, hq=32, hkv=8, d=128, T=2048,
                                   bits=4, pct=20, recent=64, steps=100, pairs=2, factor=20.0),
    # reduced-precision importance cache: 20% importance at INT4 or INT8 over a
    # 2-bit retention cache (the setting of Table 3 on the velog notes page)
    "llama2_7b_imp4": DecodeConfig("llama2_7b_imp4", batch=8, hq=32, hkv=32, d=128, T=4096,
                                   bits=2, pct=20, recent=64, steps=128, pairs=2, factor=20.0,
                                   imp_bits=4),
    "llama2_7b_imp8": DecodeConfig("llama2_7b_imp8", batch=8, hq=32, hkv=32, d=128, T=4096,
                                   bits=2, pct=20, recent=64, steps=128, pairs=2, factor=20.0,
                                   imp_bits=8),
    # per-channel key quantization over 64-token tiles with the fp16 token
    # buffer, 20% importance (the setting of appendix C on the paperlayer
    # page), on the Llama-2-7B layer shape
    "llama2_7b_kchan": DecodeConfig("llama2_7b_kchan", batch=8, hq=32, hkv=32, d=128, T=4096,
                                    bits=4, pct=20, recent=64, steps=128, pairs=2, factor=20.0,
                                    key_tile=64),
}

CKV_CONFIGS = {
    "criticalkv_32k": CriticalKVConfig("criticalkv_32k", H=32, d=128, hidden=4096, T=32768,
                                       pct=20, alpha=0.5, sigma=3.0),
}

# stream ids keep the draws of different arrays independent
_S_OUTLIER, _S_PREFILL, _S_ACC0, _S_DECODE, _S_CKV = 1, 2, 3, 4, 5


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(x) for x in key]))


def outlier_channels(cfg: DecodeConfig, seed: int) -> np.ndarray:
    """[hkv, 2*pairs] int64 channel indices, RoPE-duplicated pairs {c, c+d/2}."""
    out = np.empty((cfg.hkv, 2 * cfg.pairs), np.int64)
    half = cfg.d // 2
    for g in range(cfg.hkv):
        c = _rng(seed, _S_OUTLIER, g).choice(half, size=cfg.pairs, replace=False)
        out[g] = np.concatenate([c, c + half])
    return out


def _normal16(rng, shape, scale_ch=None, factor=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale_ch is not None and len(scale_ch):
        x[..., scale_ch] *= np.float32(factor)
    return x.astype(np.float16)


def unit_prefill(cfg: DecodeConfig, seed: int, n: int, g: int, ch=None):
    """Prompt q [rep,T,d], k [T,d], v [T,d] (fp16) for sequence n, kv head g."""
    if ch is None:
        ch = outlier_channels(cfg, seed)[g]
    rng = _rng(seed, _S_PREFILL, n, g)
    q = _normal16(rng, (cfg.rep, cfg.T, cfg.d), ch, cfg.factor)
    k = _normal16(rng, (cfg.T, cfg.d), ch, cfg.factor)
    v = _normal16(rng, (cfg.T, cfg.d))
    return q, k, v


def unit_acc0(cfg: DecodeConfig, seed: int, n: int, g: int) -> np.ndarray:
    """Stand-in prefill heavy-hitter scores [T] fp32 (see module docstring)."""
    rng = _rng(seed, _S_ACC0, n, g)
    a = rng.lognormal(mean=0.0, sigma=2.0, size=cfg.T)
    if cfg.T > 0:
        a *= cfg.rep * cfg.T / a.sum()
    a = np.round(a * 1024.0) / 1024.0
    a[rng.random(cfg.T) < 0.05] = 0.0
    return a.astype(np.float32)


def unit_decode(cfg: DecodeConfig, seed: int, step: int, n: int, g: int, ch=None):
    """New-token q [rep,d], k [d], v [d] (fp16) of decode step `step`."""
    if ch is None:
        ch = outlier_channels(cfg, seed)[g]
    rng = _rng(seed, _S_DECODE, step, n, g)
    q = _normal16(rng, (cfg.rep, cfg.d), ch, cfg.factor)
    k = _normal16(rng, (cfg.d,), ch, cfg.factor)
    v = _normal16(rng, (cfg.d,))
    return q, k, v


def prefill_tensors(cfg: DecodeConfig, seed: int):
    """Full prompt tensors: q [n,hq,T,d], k/v [n,hkv,T,d] fp16, acc0 [n,hkv,T] fp32."""
    chs = outlier_channels(cfg, seed)
    q = np.empty((cfg.batch, cfg.hq, cfg.T, cfg.d), np.float16)
    k = np.empty((cfg.batch, cfg.hkv, cfg.T, cfg.d), np.float16)
    v = np.empty_like(k)
    acc0 = np.empty((cfg.batch, cfg.hkv, cfg.T), np.float32)
    r = cfg.rep
    for n in range(cfg.batch):
        for g in range(cfg.hkv):
            qu, ku, vu = unit_prefill(cfg, seed, n, g, chs[g])
            q[n, g * r:(g + 1) * r] = qu
            k[n, g] = ku
            v[n, g] = vu
            acc0[n, g] = unit_acc0(cfg, seed, n, g)
    return q, k, v, acc0


def decode_tensors(cfg: DecodeConfig, seed: int, step: int):
    """One decode step's inputs: q [n,hq,d], k/v [n,hkv,d] fp16."""
    chs = outlier_channels(cfg, seed)
    q = np.empty((cfg.batch, cfg.hq, cfg.d), np.float16)
    k = np.empty((cfg.batch, cfg.hkv, cfg.d), np.float16)
    v = np.empty_like(k)
    r = cfg.rep
    for n in range(cfg.batch):
        for g in range(cfg.hkv):
            qu, ku, vu = unit_decode(cfg, seed, step, n, g, chs[g])
            q[n, g * r:(g + 1) * r] = qu
            k[n, g] = ku
            v[n, g] = vu
    return q, k, v


def criticalkv_inputs(cfg: CriticalKVConfig, seed: int):
    """A [H,T] fp32 (softmax of fp16 N(0, sigma^2) logits, normalised in fp64),
    V [H,T,d] fp16 ~ N(0,1), W_O [H*d, hidden] fp16 ~ N(0, 1/hidden).

    The softmax here only shapes a synthetic attention distribution (it is
    the stated recipe for the input, not a step of the selector)."""
    rng = _rng(seed, _S_CKV)
    logits = (rng.standard_normal((cfg.H, cfg.T), dtype=np.float32)
              * np.float32(cfg.sigma)).astype(np.float16).astype(np.float64)
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    A = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    V = rng.standard_normal((cfg.H, cfg.T, cfg.d), dtype=np.float32).astype(np.float16)
    W = (rng.standard_normal((cfg.H * cfg.d, cfg.hidden), dtype=np.float32)
         * np.float32(1.0 / np.sqrt(cfg.hidden))).astype(np.float16)
    return A, V, W
