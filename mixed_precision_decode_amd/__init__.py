"""MiKV mixed-precision KV-cache path for AMD Instinct MI355X (gfx950).

The compute lives in libmikv.so (hand-written HIP kernels behind the C
interface of include/mikv.h); this package is its ctypes binding plus the
seeded synthetic workloads (synth.py). There is no CPU fallback: calling an
entry point without the built library raises.
"""
from ._lib import (  # noqa: F401
    Cache, Dims, MikvError, lib,
    mikv_abi_version, mikv_status_str,
    mikv_balance_workspace, mikv_balance_prefill,
    mikv_quantize_tokens,
    mikv_decode_attn_workspace, mikv_decode_attn, mikv_decode_step,
    mikv_h2o_workspace, mikv_h2o_update_select,
    mikv_criticalkv_workspace, mikv_criticalkv_select,
)
