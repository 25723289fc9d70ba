"""C interface checks that need no GPU: the library loads, exports every
function include/mikv.h declares, and rejects invalid arguments on the host
with the documented status before anything is enqueued."""
import ctypes as C
import os
import re

import pytest

from mixed_precision_decode_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20   # never dereferenced: validation fails before any launch


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from mixed_precision_decode_amd import build_lib
        build_lib.build()
    return L.lib()


def _header_functions():
    txt = open(os.path.join(ROOT, "include", "mikv.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mikv_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_function(lib):
    names = _header_functions()
    assert len(names) == 20, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L._SIGS)


def test_abi_version_and_status_text(lib):
    assert lib.mikv_abi_version() == 4
    for s in range(8):
        assert len(L.mikv_status_str(s)) > 0
    assert L.mikv_status_str(99) == "unknown status"


def _dims(**kw):
    d = dict(batch=2, hq=8, hkv=2, d=128, group=64, bits=4, cap16=11, capq=100)
    d.update(kw)
    return L.Dims(**d)


def _cache():
    return L.MikvCache(*([FAKE] * 10))


def test_decode_attn_validation(lib):
    c = _cache()
    good = _dims()
    ws_need = lib.mikv_decode_attn_workspace(C.byref(good.c()), 80)
    assert ws_need > 0
    call = lambda dims, length=50, ws_bytes=ws_need, cache=c, q=FAKE: lib.mikv_decode_attn(
        C.byref(dims.c()), C.byref(cache), length, q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        ws_bytes, None)
    assert call(_dims(hq=7)) == L.MIKV_ERR_SHAPE
    assert call(_dims(d=96)) == L.MIKV_ERR_UNSUPPORTED
    assert call(_dims(bits=3)) == L.MIKV_ERR_UNSUPPORTED
    assert call(_dims(group=32)) == L.MIKV_ERR_UNSUPPORTED
    assert call(good, q=None) == L.MIKV_ERR_NULL
    assert call(good, length=10) == L.MIKV_ERR_SHAPE            # len < cap16
    assert call(good, length=112) == L.MIKV_ERR_CAPACITY        # len - cap16 > capq
    assert call(good, ws_bytes=16) == L.MIKV_ERR_WORKSPACE
    bad = _cache()
    bad.kq = None
    assert call(good, cache=bad) == L.MIKV_ERR_NULL
    mis = _cache()
    mis.k16 = FAKE + 2
    assert call(good, cache=mis) == L.MIKV_ERR_SHAPE            # 16-byte alignment


def test_decode_attn_timed_validation(lib):
    c = _cache()
    good = _dims()
    ws_need = lib.mikv_decode_attn_workspace(C.byref(good.c()), 80)
    call = lambda dims=good, length=50, ws_bytes=ws_need, ev0=FAKE, ev1=FAKE: lib.mikv_decode_attn_timed(
        C.byref(dims.c()), C.byref(c), length, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        ws_bytes, None, ev0, ev1)
    assert call(ev0=None) == L.MIKV_ERR_NULL
    assert call(ev1=None) == L.MIKV_ERR_NULL
    assert call(_dims(hq=7)) == L.MIKV_ERR_SHAPE
    assert call(length=112) == L.MIKV_ERR_CAPACITY
    assert call(ws_bytes=16) == L.MIKV_ERR_WORKSPACE


def test_prefill_scores_validation(lib):
    good = _dims()
    T = 300
    need = lib.mikv_prefill_scores_workspace(C.byref(good.c()), T)
    assert need == 2 * 8 * T * 4                      # log-sum-exp per query row and head
    call = lambda dims=good, T=T, q=FAKE, k=FAKE, acc=FAKE, ws_bytes=need: lib.mikv_prefill_scores(
        C.byref(dims.c()), T, q, k, acc, FAKE, ws_bytes, None)
    assert call(_dims(hq=7)) == L.MIKV_ERR_SHAPE
    assert call(_dims(d=96)) == L.MIKV_ERR_UNSUPPORTED
    assert call(q=None) == L.MIKV_ERR_NULL
    assert call(k=None) == L.MIKV_ERR_NULL
    assert call(acc=None) == L.MIKV_ERR_NULL
    assert call(q=FAKE + 2) == L.MIKV_ERR_SHAPE           # 16-byte alignment
    assert call(T=-1) == L.MIKV_ERR_SHAPE
    assert call(ws_bytes=need - 1) == L.MIKV_ERR_WORKSPACE
    assert call(T=0, q=None, k=None, acc=None) == L.MIKV_OK    # nothing to do, nothing enqueued


def test_read_probe_validation(lib):
    call = lambda p=FAKE, nbytes=1 << 20, blocks=8, sink=FAKE: lib.mikv_read_probe(p, nbytes, blocks, sink, None)
    assert call(p=None) == L.MIKV_ERR_NULL
    assert call(sink=None) == L.MIKV_ERR_NULL
    assert call(p=FAKE + 4) == L.MIKV_ERR_SHAPE
    assert call(nbytes=(1 << 20) + 8) == L.MIKV_ERR_SHAPE
    assert call(blocks=0) == L.MIKV_ERR_SHAPE
    assert call(nbytes=0, p=None, sink=None) == L.MIKV_OK


def test_decode_step_validation(lib):
    c = _cache()
    good = _dims()
    need = lib.mikv_decode_attn_workspace(C.byref(good.c()), 80)
    call = lambda dims=good, length=50, recent=4, heavy=6, ws_bytes=need, q=FAKE: lib.mikv_decode_step(
        C.byref(dims.c()), C.byref(c), length, recent, heavy, q, FAKE, FAKE, FAKE, FAKE, FAKE, None,
        FAKE, ws_bytes, None)
    assert call(q=None) == L.MIKV_ERR_NULL
    assert call(recent=5) == L.MIKV_ERR_SHAPE
    assert call(length=10) == L.MIKV_ERR_SHAPE
    assert call(length=111) == L.MIKV_ERR_CAPACITY     # demotion would need slot 100
    assert call(ws_bytes=16) == L.MIKV_ERR_WORKSPACE
    assert call(_dims(bits=8)) == L.MIKV_ERR_UNSUPPORTED


def test_importance_codes_validation(lib):
    """imp_bits: 16 or 0 = fp16 importance tier, 8 or 4 = codes (with groups
    of d/2 and the kimp/vimp/kimpsz/vimpsz pointers); anything else is
    refused before a launch."""
    c = _cache()
    need = lib.mikv_decode_attn_workspace(C.byref(_dims(imp_bits=8).c()), 80)
    assert need > 0
    call = lambda dims, cache=c: lib.mikv_decode_attn(
        C.byref(dims.c()), C.byref(cache), 50, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None)
    assert call(_dims(imp_bits=6)) == L.MIKV_ERR_UNSUPPORTED
    assert call(_dims(imp_bits=2)) == L.MIKV_ERR_UNSUPPORTED
    assert call(_dims(imp_bits=8, group=128)) == L.MIKV_ERR_UNSUPPORTED
    # codes tier without its pointers; an fp16 tier may leave them NULL
    no_imp = L.MikvCache(*([FAKE] * 10 + [0] * 4))
    assert call(_dims(imp_bits=8), no_imp) == L.MIKV_ERR_NULL
    no16 = L.MikvCache(*([0, 0] + [FAKE] * 12))
    assert call(_dims(imp_bits=16), no16) == L.MIKV_ERR_NULL
    step = lambda dims, cache: lib.mikv_decode_step(
        C.byref(dims.c()), C.byref(cache), 50, 4, 6, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, None)
    assert step(_dims(imp_bits=4), no_imp) == L.MIKV_ERR_NULL
    assert step(_dims(imp_bits=4), no16) == L.MIKV_ERR_WORKSPACE  # checks pass up to the workspace
    h2o = lambda dims, cache: lib.mikv_h2o_update_select(
        C.byref(dims.c()), C.byref(cache), 50, 4, 6, FAKE, None, None, None, 0, None)
    assert h2o(_dims(imp_bits=8), no_imp) == L.MIKV_ERR_NULL


def test_key_tile_validation(lib):
    """key_tile: 0 = per-token keys, 64 = per-channel key tiles (fp16
    importance tier, capq a whole number of tiles, the kcsz/kbuf/vbuf/posbuf
    pointers; ksz may then be NULL); anything else is refused before a
    launch."""
    kt = _dims(key_tile=64, capq=128)
    need = lib.mikv_decode_attn_workspace(C.byref(kt.c()), 80)
    assert need > 0
    full = L.MikvCache(*([FAKE] * 18))
    call = lambda dims, cache=full: lib.mikv_decode_attn(
        C.byref(dims.c()), C.byref(cache), 50, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None)
    assert call(_dims(key_tile=32, capq=128)) == L.MIKV_ERR_UNSUPPORTED
    assert call(_dims(key_tile=1, capq=128)) == L.MIKV_ERR_UNSUPPORTED
    assert call(_dims(key_tile=64, capq=100)) == L.MIKV_ERR_SHAPE
    assert call(_dims(key_tile=64, capq=128, imp_bits=8)) == L.MIKV_ERR_UNSUPPORTED
    no_kt = L.MikvCache(*([FAKE] * 14 + [0] * 4))
    assert call(kt, no_kt) == L.MIKV_ERR_NULL
    for i in range(4):  # each of kcsz, kbuf, vbuf, posbuf
        ptrs = [FAKE] * 18
        ptrs[14 + i] = 0
        assert call(kt, L.MikvCache(*ptrs)) == L.MIKV_ERR_NULL, i
    mis = [FAKE] * 18
    mis[15] = FAKE + 4  # kbuf not 16-byte aligned
    assert call(kt, L.MikvCache(*mis)) == L.MIKV_ERR_SHAPE
    # per-channel keys need no per-token key scales: a NULL ksz passes the
    # cache checks (the call then stops at the missing workspace)
    no_ksz = [FAKE] * 18
    no_ksz[7] = 0
    assert lib.mikv_decode_attn(C.byref(kt.c()), C.byref(L.MikvCache(*no_ksz)), 50, FAKE, FAKE, FAKE, FAKE,
                                FAKE, FAKE, None, need, None) == L.MIKV_ERR_WORKSPACE
    assert call(_dims(capq=128), L.MikvCache(*no_ksz)) == L.MIKV_ERR_NULL  # per-token keys need ksz
    step = lambda dims, cache: lib.mikv_decode_step(
        C.byref(dims.c()), C.byref(cache), 50, 4, 6, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, None)
    assert step(kt, no_kt) == L.MIKV_ERR_NULL
    assert step(kt, full) == L.MIKV_ERR_WORKSPACE
    h2o = lambda dims, cache: lib.mikv_h2o_update_select(
        C.byref(dims.c()), C.byref(cache), 50, 4, 6, FAKE, None, None, None, 0, None)
    assert h2o(kt, no_kt) == L.MIKV_ERR_NULL
    assert h2o(_dims(key_tile=64, capq=96), full) == L.MIKV_ERR_SHAPE


def test_perturbation_validation(lib):
    need = lib.mikv_perturbation_workspace(4, 100, 128, 256)
    assert need > 0 and lib.mikv_perturbation_workspace(4, 100, 96, 256) == 0
    call = lambda keep=FAKE, n_keep=5, o_hat=None, H=4, T=100, d=128, hidden=256, ws_bytes=need, q=FAKE: \
        lib.mikv_output_perturbation(q, FAKE, FAKE, FAKE, keep, n_keep, o_hat, H, T, d, hidden, None, None,
                                     FAKE, FAKE, FAKE, ws_bytes, None)
    assert call(q=None) == L.MIKV_ERR_NULL
    assert call(keep=None) == L.MIKV_ERR_NULL            # neither keep nor o_hat
    assert call(o_hat=FAKE) == L.MIKV_ERR_NULL           # both
    assert call(d=96) == L.MIKV_ERR_UNSUPPORTED
    assert call(n_keep=0) == L.MIKV_ERR_SHAPE
    assert call(n_keep=101) == L.MIKV_ERR_SHAPE
    assert call(T=0) == L.MIKV_ERR_SHAPE
    assert call(T=(1 << 23)) == L.MIKV_ERR_SHAPE         # T*d*2 >= 2^31
    assert call(ws_bytes=8) == L.MIKV_ERR_WORKSPACE


def test_decode_step_noalloc_validation(lib):
    """The fixed-scratch decode step checks like mikv_decode_step and
    rejects shapes whose partial results exceed its scratch before any
    HIP call."""
    c = _cache()
    good = _dims()
    assert lib.mikv_decode_step_noalloc_limit() == 16 << 20
    call = lambda dims=good, length=50, recent=4, heavy=6, q=FAKE: lib.mikv_decode_step_noalloc(
        C.byref(dims.c()), C.byref(c), length, recent, heavy, q, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert call(q=None) == L.MIKV_ERR_NULL
    assert call(recent=5) == L.MIKV_ERR_SHAPE
    assert call(length=10) == L.MIKV_ERR_SHAPE
    assert call(length=111) == L.MIKV_ERR_CAPACITY
    assert call(_dims(bits=8)) == L.MIKV_ERR_UNSUPPORTED
    big = _dims(batch=64, hq=32, hkv=32, cap16=4097, capq=100)
    need = lib.mikv_decode_attn_workspace(C.byref(big.c()), 4097 + 50)
    assert need > lib.mikv_decode_step_noalloc_limit()
    assert call(big, length=4097 + 50, recent=64, heavy=4032) == L.MIKV_ERR_SCRATCH


def test_h2o_validation(lib):
    c = _cache()
    dims = _dims()
    dec = lambda recent, heavy, length=50, p16=FAKE: lib.mikv_h2o_update_select(
        C.byref(dims.c()), C.byref(c), length, recent, heavy, p16, None, None, None, 0, None)
    assert dec(4, 7) == L.MIKV_ERR_SHAPE        # heavy + recent != cap16 - 1
    assert dec(-1, 11) == L.MIKV_ERR_SHAPE
    assert dec(4, 6, length=112) == L.MIKV_ERR_CAPACITY
    assert dec(4, 6, p16=None) == L.MIKV_ERR_NULL  # neither mode
    src = L.MikvPrefillSrc(FAKE, FAKE, FAKE, None, 40)
    pre = lambda length, ws_bytes, s=src: lib.mikv_h2o_update_select(
        C.byref(dims.c()), C.byref(c), length, 4, 6, None, C.byref(s), None, FAKE, ws_bytes, None)
    need = lib.mikv_h2o_workspace(C.byref(dims.c()), 40)
    assert pre(39, need) == L.MIKV_ERR_SHAPE      # len != src.T
    assert pre(40, need - 1) == L.MIKV_ERR_WORKSPACE
    small = L.MikvPrefillSrc(FAKE, FAKE, FAKE, None, 9)
    assert pre(9, need, small) == L.MIKV_ERR_SHAPE  # T < B
    mis_b = L.MikvPrefillSrc(FAKE, FAKE, FAKE, FAKE + 4, 40)
    assert pre(40, need, mis_b) == L.MIKV_ERR_SHAPE  # balancer not 16-byte aligned
    tight = _dims(capq=20)
    assert lib.mikv_h2o_update_select(C.byref(tight.c()), C.byref(c), 40, 4, 6, None,
                                      C.byref(src), None, FAKE, need, None) == L.MIKV_ERR_CAPACITY


def test_balance_quantize_validation(lib):
    dims = _dims()
    need = lib.mikv_balance_workspace(C.byref(dims.c()), 64)
    assert need > 0
    bal = lambda T, q=FAKE, b=FAKE, ws_bytes=need: lib.mikv_balance_prefill(
        C.byref(dims.c()), T, q, FAKE, b, None, FAKE, ws_bytes, None)
    assert bal(-1) == L.MIKV_ERR_SHAPE
    assert bal(64, q=None) == L.MIKV_ERR_NULL
    assert bal(64, b=None) == L.MIKV_ERR_NULL
    assert bal(64, ws_bytes=need - 1) == L.MIKV_ERR_WORKSPACE
    q = lambda n, d, g, bits, x=FAKE: lib.mikv_quantize_tokens(x, None, n, d, g, bits, FAKE, FAKE, None)
    assert q(-1, 128, 64, 4) == L.MIKV_ERR_SHAPE
    assert q(5, 128, 48, 4) == L.MIKV_ERR_SHAPE
    assert q(5, 96, 48, 4) == L.MIKV_ERR_UNSUPPORTED
    assert q(5, 128, 64, 8) == L.MIKV_ERR_UNSUPPORTED
    assert q(5, 128, 64, 4, x=None) == L.MIKV_ERR_NULL
    assert q(0, 128, 64, 4, x=None) == L.MIKV_OK      # empty input enqueues nothing


def test_criticalkv_validation(lib):
    need = lib.mikv_criticalkv_workspace(4, 100, 128, 256)
    assert need > 0
    ck = lambda H=4, T=100, d=128, hidden=256, budget=20, alpha=0.5, ws_bytes=need, A=FAKE: \
        lib.mikv_criticalkv_select(A, FAKE, FAKE, H, T, d, hidden, budget, alpha, FAKE, None,
                                   FAKE, ws_bytes, None)
    assert ck(A=None) == L.MIKV_ERR_NULL
    assert ck(d=64) == L.MIKV_ERR_UNSUPPORTED
    assert ck(hidden=200) == L.MIKV_ERR_UNSUPPORTED
    assert ck(budget=0) == L.MIKV_ERR_SHAPE
    assert ck(budget=101) == L.MIKV_ERR_SHAPE
    assert ck(alpha=1.5) == L.MIKV_ERR_SHAPE
    assert ck(alpha=float("nan")) == L.MIKV_ERR_SHAPE
    assert ck(ws_bytes=need - 1) == L.MIKV_ERR_WORKSPACE


def test_workspace_queries(lib):
    dims = _dims()
    a = lib.mikv_decode_attn_workspace(C.byref(dims.c()), 1000)
    b = lib.mikv_decode_attn_workspace(C.byref(dims.c()), 4000)
    assert 0 < a <= b
    assert lib.mikv_decode_attn_workspace(C.byref(dims.c()), 5) == 0   # max_len < cap16


def _no_device():
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_device(), reason="launches with fake pointers: only where no GPU is visible")
@pytest.mark.parametrize("batch,hq,hkv,d,bits,group,cap16", [
    (8, 32, 32, 128, 4, 64, 820), (1, 32, 8, 128, 2, 64, 3277), (64, 32, 8, 128, 4, 64, 410),
    (1, 1, 1, 64, 4, 32, 52), (3, 9, 3, 64, 2, 64, 17), (2, 16, 2, 128, 4, 128, 1),
    (256, 1, 1, 64, 4, 32, 52), (1, 64, 1, 128, 4, 64, 5000),
])
def test_workspace_bound_covers_every_length(lib, batch, hq, hkv, d, bits, group, cap16):
    """The workspace bound for max_len serves every length up to max_len: a
    call with exactly that many bytes passes the workspace check and fails
    only at the launch (no device here)."""
    max_len = cap16 + 40000
    dims = L.Dims(batch=batch, hq=hq, hkv=hkv, d=d, group=group, bits=bits, cap16=cap16, capq=max_len)
    need = lib.mikv_decode_attn_workspace(C.byref(dims.c()), max_len)
    assert need > 0
    c = _cache()
    for length in sorted({cap16, cap16 + 1, cap16 + 7, cap16 + 600, cap16 + 4097, max_len - 1, max_len}):
        st = lib.mikv_decode_attn(C.byref(dims.c()), C.byref(c), length, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, need, None)
        assert st == L.MIKV_ERR_HIP, (length, st)
        st = lib.mikv_decode_step(C.byref(dims.c()), C.byref(c), length, 0, cap16 - 1, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, None, FAKE, need, None)
        assert st in (L.MIKV_ERR_HIP, L.MIKV_ERR_CAPACITY), (length, st)


def test_tier_offsets_limit(lib):
    """The decode kernels address one (sequence, kv head) tier with 32-bit
    byte offsets: larger per-unit tiers are rejected before any launch."""
    c = _cache()
    big = _dims(capq=1 << 27)            # 2^27 slots * 64 B = 2^33 B of INT4 codes
    assert lib.mikv_decode_attn(C.byref(big.c()), C.byref(c), 50, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, 1 << 40, None) == L.MIKV_ERR_SHAPE
    big16 = _dims(cap16=1 << 23, capq=100)   # 2^23 slots * 256 B = 2^31 B of fp16 rows
    assert lib.mikv_decode_attn(C.byref(big16.c()), C.byref(c), (1 << 23) + 5, FAKE, FAKE, FAKE, FAKE,
                                FAKE, FAKE, FAKE, 1 << 40, None) == L.MIKV_ERR_SHAPE


def test_header_is_plain_c(lib, tmp_path):
    """include/mikv.h compiles as C99 on its own (no HIP or C++ headers), and
    a C program linked against the library gets the documented statuses
    from host-side validation."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "abi_check.c"
    src.write_text(r'''
#include <stdio.h>
#include "mikv.h"
int main(void) {
  mikv_dims d = {2, 8, 2, 128, 64, 4, 11, 100};
  mikv_dims bad = d;
  bad.hq = 7;
  int fails = 0;
  if (mikv_abi_version() != MIKV_ABI_VERSION) fails++;
  if (mikv_decode_attn_workspace(&d, 80) == 0) fails++;
  if (mikv_decode_attn(&bad, NULL, 50, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) != MIKV_ERR_SHAPE) fails++;
  if (mikv_decode_attn(&d, NULL, 50, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) != MIKV_ERR_NULL) fails++;
  if (mikv_prefill_scores(&d, 0, NULL, NULL, NULL, NULL, 0, NULL) != MIKV_OK) fails++;
  if (mikv_read_probe(NULL, 16, 1, NULL, NULL) != MIKV_ERR_NULL) fails++;
  printf("%s %d\n", mikv_status_str(MIKV_ERR_CAPACITY), fails);
  return fails;
}
''')
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(L.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"), str(src),
           "-o", str(exe), "-L", libdir, "-lmikv", "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.stdout, r.stderr)
    assert r.stdout.strip().endswith(" 0")
