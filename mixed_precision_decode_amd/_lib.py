"""ctypes binding of libmikv.so (see include/mikv.h for every contract).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers and the current HIP stream are passed to the
C entry point of the same name, and a non-OK status raises MikvError. All
computation happens in the library's HIP kernels. fp16 tensors may be
torch.float16 or torch.int16/uint16 bit patterns.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmikv.so")

MIKV_OK, MIKV_ERR_NULL, MIKV_ERR_SHAPE, MIKV_ERR_UNSUPPORTED = 0, 1, 2, 3
MIKV_ERR_CAPACITY, MIKV_ERR_WORKSPACE, MIKV_ERR_HIP, MIKV_ERR_SCRATCH = 4, 5, 6, 7

_vp, _sz, _i32, _i64, _f64 = C.c_void_p, C.c_size_t, C.c_int32, C.c_int64, C.c_double


class MikvDims(C.Structure):
    _fields_ = [(n, _i32) for n in ("batch", "hq", "hkv", "d", "group", "bits", "cap16", "capq",
                                     "imp_bits", "key_tile")]


class MikvCache(C.Structure):
    _fields_ = [(n, _vp) for n in ("k16", "v16", "pos16", "acc16", "free16",
                                   "kq", "vq", "ksz", "vsz", "posq",
                                   "kimp", "vimp", "kimpsz", "vimpsz",
                                   "kcsz", "kbuf", "vbuf", "posbuf")]


class MikvPrefillSrc(C.Structure):
    _fields_ = [("k", _vp), ("v", _vp), ("acc0", _vp), ("b", _vp), ("T", _i32)]


class MikvError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"mikv status {status}: {text}")
        self.status = status


_lib = None

_SIGS = {
    "mikv_status_str": (C.c_char_p, [C.c_int]),
    "mikv_abi_version": (C.c_int, []),
    "mikv_balance_workspace": (_sz, [C.POINTER(MikvDims), _i32]),
    "mikv_balance_prefill": (C.c_int, [C.POINTER(MikvDims), _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mikv_prefill_scores_workspace": (_sz, [C.POINTER(MikvDims), _i32]),
    "mikv_prefill_scores": (C.c_int, [C.POINTER(MikvDims), _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mikv_read_probe": (C.c_int, [_vp, _sz, _i32, _vp, _vp]),
    "mikv_quantize_tokens": (C.c_int, [_vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp]),
    "mikv_decode_attn_workspace": (_sz, [C.POINTER(MikvDims), _i32]),
    "mikv_decode_attn": (C.c_int, [C.POINTER(MikvDims), C.POINTER(MikvCache), _i32, _vp, _vp, _vp,
                                   _vp, _vp, _vp, _vp, _sz, _vp]),
    "mikv_decode_attn_timed": (C.c_int, [C.POINTER(MikvDims), C.POINTER(MikvCache), _i32, _vp, _vp, _vp,
                                         _vp, _vp, _vp, _vp, _sz, _vp, _vp, _vp]),
    "mikv_decode_step": (C.c_int, [C.POINTER(MikvDims), C.POINTER(MikvCache), _i32, _i32, _i32, _vp,
                                   _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mikv_decode_step_noalloc_limit": (_sz, []),
    "mikv_decode_step_noalloc": (C.c_int, [C.POINTER(MikvDims), C.POINTER(MikvCache), _i32, _i32, _i32,
                                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "mikv_h2o_workspace": (_sz, [C.POINTER(MikvDims), _i32]),
    "mikv_h2o_update_select": (C.c_int, [C.POINTER(MikvDims), C.POINTER(MikvCache), _i32, _i32, _i32,
                                         _vp, C.POINTER(MikvPrefillSrc), _vp, _vp, _sz, _vp]),
    "mikv_perturbation_workspace": (_sz, [_i32, _i32, _i32, _i32]),
    "mikv_output_perturbation": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                           _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mikv_criticalkv_workspace": (_sz, [_i32, _i32, _i32, _i32]),
    "mikv_criticalkv_select": (C.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f64, _vp, _vp,
                                         _vp, _sz, _vp]),
}


def lib() -> C.CDLL:
    """The loaded library. Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _check(status: int):
    if status != MIKV_OK:
        raise MikvError(status, lib().mikv_status_str(status).decode())


@dataclasses.dataclass
class Dims:
    batch: int
    hq: int
    hkv: int
    d: int
    group: int
    bits: int
    cap16: int
    capq: int
    imp_bits: int = 16
    key_tile: int = 0

    def c(self) -> MikvDims:
        key = tuple(int(getattr(self, f.name)) for f in dataclasses.fields(self))
        cached = self.__dict__.get("_c")
        if cached is None or cached[0] != key:
            cached = (key, MikvDims(*key))
            self.__dict__["_c"] = cached
        return cached[1]


def _ptr(t, dtype=None, shape=None, name="tensor", optional=False):
    import torch
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None:
        ok = (torch.float16, torch.int16, torch.uint16) if dtype == "f16" else (dtype,)
        if t.dtype not in ok:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _i32t():
    import torch
    return torch.int32


def _f32t():
    import torch
    return torch.float32


def mikv_status_str(status: int) -> str:
    return lib().mikv_status_str(status).decode()


def mikv_abi_version() -> int:
    return lib().mikv_abi_version()


def mikv_balance_workspace(dims: Dims, T: int) -> int:
    return lib().mikv_balance_workspace(C.byref(dims.c()), T)


def mikv_decode_attn_workspace(dims: Dims, max_len: int) -> int:
    return lib().mikv_decode_attn_workspace(C.byref(dims.c()), max_len)


def mikv_h2o_workspace(dims: Dims, max_T: int) -> int:
    return lib().mikv_h2o_workspace(C.byref(dims.c()), max_T)


def mikv_criticalkv_workspace(H: int, T: int, d: int, hidden: int) -> int:
    return lib().mikv_criticalkv_workspace(H, T, d, hidden)


def mikv_balance_prefill(dims: Dims, T: int, q, k, b, kb=None, ws=None, stream=None):
    n, hq, hkv, d = dims.batch, dims.hq, dims.hkv, dims.d
    _check(lib().mikv_balance_prefill(
        C.byref(dims.c()), T,
        _ptr(q, "f16", (n, hq, T, d), "q"), _ptr(k, "f16", (n, hkv, T, d), "k"),
        _ptr(b, _f32t(), (n, hkv, d), "b"), _ptr(kb, "f16", (n, hkv, T, d), "kb", optional=True),
        _ptr(ws, name="ws", optional=True), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def mikv_prefill_scores_workspace(dims: Dims, T: int) -> int:
    return lib().mikv_prefill_scores_workspace(C.byref(dims.c()), T)


def mikv_prefill_scores(dims: Dims, T: int, q, k, acc0, ws, stream=None):
    n, hq, hkv, d = dims.batch, dims.hq, dims.hkv, dims.d
    _check(lib().mikv_prefill_scores(
        C.byref(dims.c()), T,
        _ptr(q, "f16", (n, hq, T, d), "q"), _ptr(k, "f16", (n, hkv, T, d), "k"),
        _ptr(acc0, _f32t(), (n, hkv, T), "acc0"),
        _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream)))


def mikv_read_probe(buf, blocks: int, sink, stream=None):
    """Streaming read of the whole of `buf` (measurement helper)."""
    _check(lib().mikv_read_probe(_ptr(buf, name="buf"), buf.numel() * buf.element_size(), blocks,
                                 _ptr(sink, None, (blocks,), "sink"), _stream(stream)))


def mikv_quantize_tokens(x, rows, codes, sz, group: int, bits: int, stream=None):
    """Row r of codes/sz quantizes row rows[r] of x (rows given) or row r
    (rows None); x holds whole rows of d channels."""
    n_rows, cb = codes.shape
    d = x.shape[-1]
    if x.numel() % d != 0 or (rows is None and x.numel() < n_rows * d):
        raise ValueError(f"x: {x.numel()} elements do not hold {n_rows} rows of {d}")
    _check(lib().mikv_quantize_tokens(
        _ptr(x, "f16", None, "x"), _ptr(rows, _i32t(), (n_rows,), "rows", optional=True),
        n_rows, d, group, bits,
        _ptr(codes, None, (n_rows, d * bits // 8), "codes"),
        _ptr(sz, "f16", (n_rows, d // group, 2), "sz"), _stream(stream)))


class Cache:
    """Device tensors of one two-tier cache (layout of include/mikv.h). With
    dims.imp_bits 8 or 4 the importance tier is kimp/vimp codes with
    kimpsz/vimpsz (scale, zero), and k16/v16 are not allocated. With
    dims.key_tile 64 the retained keys are per-channel tiles (kcsz in place
    of ksz) with the fp16 buffer kbuf/vbuf/posbuf."""

    def __init__(self, dims: Dims, device="cuda"):
        import torch
        n, g, d, c16, cq = dims.batch, dims.hkv, dims.d, dims.cap16, dims.capq
        self.dims = dims
        ib = dims.imp_bits or 16
        self.imp_bits = ib
        if ib == 16:
            self.k16 = torch.zeros((n, g, c16, d), dtype=torch.float16, device=device)
            self.v16 = torch.zeros_like(self.k16)
        else:
            self.kimp = torch.zeros((n, g, c16, d * ib // 8), dtype=torch.uint8, device=device)
            self.vimp = torch.zeros_like(self.kimp)
            self.kimpsz = torch.zeros((n, g, c16, d // dims.group, 2), dtype=torch.float16, device=device)
            self.vimpsz = torch.zeros_like(self.kimpsz)
        self.pos16 = torch.full((n, g, c16), -1, dtype=torch.int32, device=device)
        self.acc16 = torch.zeros((n, g, c16), dtype=torch.float32, device=device)
        self.free16 = torch.zeros((n, g), dtype=torch.int32, device=device)
        cb = d * dims.bits // 8
        self.kq = torch.zeros((n, g, cq, cb), dtype=torch.uint8, device=device)
        self.vq = torch.zeros_like(self.kq)
        self.vsz = torch.zeros((n, g, cq, d // dims.group, 2), dtype=torch.float16, device=device)
        self.posq = torch.full((n, g, cq), -1, dtype=torch.int32, device=device)
        self.key_tile = dims.key_tile
        if dims.key_tile:
            kt = dims.key_tile
            self.kcsz = torch.zeros((n, g, cq // kt, d, 2), dtype=torch.float16, device=device)
            self.kbuf = torch.zeros((n, g, kt, d), dtype=torch.float16, device=device)
            self.vbuf = torch.zeros_like(self.kbuf)
            self.posbuf = torch.full((n, g, kt), -1, dtype=torch.int32, device=device)
        else:
            self.ksz = torch.zeros_like(self.vsz)

    def c(self) -> MikvCache:
        if getattr(self, "_c", None) is None:
            self._c = MikvCache(*(getattr(self, f).data_ptr() if hasattr(self, f) else None
                                  for f, _ in MikvCache._fields_))
        return self._c

    COMMON = ("pos16", "acc16", "free16", "kq", "vq", "ksz", "vsz", "posq")
    NAMES = ("k16", "v16") + COMMON
    IMP_NAMES = ("kimp", "vimp", "kimpsz", "vimpsz") + COMMON

    KT_NAMES = ("k16", "v16", "pos16", "acc16", "free16", "kq", "vq", "vsz", "posq",
                "kcsz", "kbuf", "vbuf", "posbuf")

    @property
    def names(self):
        if self.key_tile:
            return self.KT_NAMES
        return self.NAMES if self.imp_bits == 16 else self.IMP_NAMES

    def to_numpy(self) -> dict:
        out = {k: getattr(self, k).cpu().numpy() for k in self.names}
        out["group"], out["bits"], out["imp_bits"] = self.dims.group, self.dims.bits, self.imp_bits
        out["key_tile"] = self.key_tile
        return out


def mikv_decode_attn(dims: Dims, cache: Cache, length: int, q, k_new, v_new, b, o, p16, ws,
                     stream=None):
    n, hq, hkv, d = dims.batch, dims.hq, dims.hkv, dims.d
    _check(lib().mikv_decode_attn(
        C.byref(dims.c()), C.byref(cache.c()), length,
        _ptr(q, "f16", (n, hq, d), "q"), _ptr(k_new, "f16", (n, hkv, d), "k_new"),
        _ptr(v_new, "f16", (n, hkv, d), "v_new"), _ptr(b, _f32t(), (n, hkv, d), "b"),
        _ptr(o, _f32t(), (n, hq, d), "o"), _ptr(p16, _f32t(), (n, hkv, dims.cap16), "p16"),
        _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream)))


def _event(ev):
    """Raw hipEvent_t of a torch.cuda.Event created with enable_timing=True
    (torch creates the event at its first record)."""
    import torch
    if not isinstance(ev, torch.cuda.Event):
        raise ValueError("expected a torch.cuda.Event")
    if not ev.cuda_event:
        ev.record()
    return ev.cuda_event


def mikv_decode_attn_timed(dims: Dims, cache: Cache, length: int, q, k_new, v_new, b, o, p16, ws,
                           split_start, split_stop, stream=None):
    """mikv_decode_attn; split_start / split_stop (torch.cuda.Event, timing
    enabled) receive the start and end of the split kernel itself."""
    n, hq, hkv, d = dims.batch, dims.hq, dims.hkv, dims.d
    _check(lib().mikv_decode_attn_timed(
        C.byref(dims.c()), C.byref(cache.c()), length,
        _ptr(q, "f16", (n, hq, d), "q"), _ptr(k_new, "f16", (n, hkv, d), "k_new"),
        _ptr(v_new, "f16", (n, hkv, d), "v_new"), _ptr(b, _f32t(), (n, hkv, d), "b"),
        _ptr(o, _f32t(), (n, hq, d), "o"), _ptr(p16, _f32t(), (n, hkv, dims.cap16), "p16"),
        _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream),
        _event(split_start), _event(split_stop)))


def mikv_decode_step(dims: Dims, cache: Cache, length: int, recent: int, heavy: int, q, k_new, v_new,
                     b, o, p16, ws, demoted_pos=None, stream=None):
    n, hq, hkv, d = dims.batch, dims.hq, dims.hkv, dims.d
    _check(lib().mikv_decode_step(
        C.byref(dims.c()), C.byref(cache.c()), length, recent, heavy,
        _ptr(q, "f16", (n, hq, d), "q"), _ptr(k_new, "f16", (n, hkv, d), "k_new"),
        _ptr(v_new, "f16", (n, hkv, d), "v_new"), _ptr(b, _f32t(), (n, hkv, d), "b"),
        _ptr(o, _f32t(), (n, hq, d), "o"), _ptr(p16, _f32t(), (n, hkv, dims.cap16), "p16"),
        _ptr(demoted_pos, _i32t(), (n, hkv), "demoted_pos", optional=True),
        _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream)))


def mikv_decode_step_noalloc_limit() -> int:
    return lib().mikv_decode_step_noalloc_limit()


def mikv_decode_step_noalloc(dims: Dims, cache: Cache, length: int, recent: int, heavy: int, q, k_new,
                             v_new, b, o, p16, demoted_pos=None, stream=None):
    """mikv_decode_step with the library's fixed device scratch in place of
    a workspace (no allocation)."""
    n, hq, hkv, d = dims.batch, dims.hq, dims.hkv, dims.d
    _check(lib().mikv_decode_step_noalloc(
        C.byref(dims.c()), C.byref(cache.c()), length, recent, heavy,
        _ptr(q, "f16", (n, hq, d), "q"), _ptr(k_new, "f16", (n, hkv, d), "k_new"),
        _ptr(v_new, "f16", (n, hkv, d), "v_new"), _ptr(b, _f32t(), (n, hkv, d), "b"),
        _ptr(o, _f32t(), (n, hq, d), "o"), _ptr(p16, _f32t(), (n, hkv, dims.cap16), "p16"),
        _ptr(demoted_pos, _i32t(), (n, hkv), "demoted_pos", optional=True), _stream(stream)))


def mikv_h2o_update_select(dims: Dims, cache: Cache, length: int, recent: int, heavy: int,
                           p16=None, src=None, demoted_pos=None, ws=None, stream=None):
    """Decode mode: pass p16. Prefill mode: pass src = dict(k=, v=, acc0=, b=None)."""
    n, hkv, d = dims.batch, dims.hkv, dims.d
    csrc = None
    if src is not None:
        T = length
        csrc = MikvPrefillSrc(_ptr(src["k"], "f16", (n, hkv, T, d), "src.k"),
                              _ptr(src["v"], "f16", (n, hkv, T, d), "src.v"),
                              _ptr(src["acc0"], _f32t(), (n, hkv, T), "src.acc0"),
                              _ptr(src.get("b"), _f32t(), (n, hkv, d), "src.b", optional=True), T)
    _check(lib().mikv_h2o_update_select(
        C.byref(dims.c()), C.byref(cache.c()), length, recent, heavy,
        _ptr(p16, _f32t(), (n, hkv, dims.cap16), "p16", optional=True),
        None if csrc is None else C.byref(csrc),
        _ptr(demoted_pos, _i32t(), (n, hkv), "demoted_pos", optional=True),
        _ptr(ws, name="ws", optional=True), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)))


def mikv_criticalkv_select(A, V, W_O, budget: int, alpha: float, idx, score2=None, ws=None,
                           stream=None):
    H, T = A.shape
    d = V.shape[-1]
    hidden = W_O.shape[1]
    _check(lib().mikv_criticalkv_select(
        _ptr(A, _f32t(), (H, T), "A"), _ptr(V, "f16", (H, T, d), "V"),
        _ptr(W_O, "f16", (H * d, hidden), "W_O"), H, T, d, hidden, budget, float(alpha),
        _ptr(idx, _i32t(), (H, budget), "idx"),
        _ptr(score2, _f32t(), (H, T), "score2", optional=True),
        _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream)))


def mikv_perturbation_workspace(H: int, T: int, d: int, hidden: int) -> int:
    return lib().mikv_perturbation_workspace(H, T, d, hidden)


def mikv_output_perturbation(q, K, V, W_O, L_head, L_proj, ws, keep=None, o_hat=None, o=None, delta=None,
                             stream=None):
    """L_head / L_proj [H] receive ||o - o_hat||_1 in head space and after
    W_O,h; keep [H, n_keep] int32 (kept token indices) or o_hat [H, d]."""
    H, T, d = K.shape
    hidden = W_O.shape[1]
    n_keep = 0 if keep is None else keep.shape[1]
    _check(lib().mikv_output_perturbation(
        _ptr(q, "f16", (H, d), "q"), _ptr(K, "f16", (H, T, d), "K"), _ptr(V, "f16", (H, T, d), "V"),
        _ptr(W_O, "f16", (H * d, hidden), "W_O"),
        _ptr(keep, _i32t(), (H, n_keep), "keep", optional=True), n_keep,
        _ptr(o_hat, _f32t(), (H, d), "o_hat", optional=True), H, T, d, hidden,
        _ptr(o, _f32t(), (H, d), "o", optional=True), _ptr(delta, _f32t(), (H, d), "delta", optional=True),
        _ptr(L_head, _f32t(), (H,), "L_head"), _ptr(L_proj, _f32t(), (H,), "L_proj"),
        _ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream)))
