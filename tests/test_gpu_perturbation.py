"""Output-perturbation diagnostic on the device (mikv_output_perturbation)
against the oracle, and the comparison of H2O eviction, CriticalKV
selection and MiKV's mixed-precision cache on one synthetic layer (gist
CriticalKV, theoretical framework: L = ||o - o_hat||_1).

The device's delta = o - o_hat is checked against the oracle's to the
attention tolerance (2e-3 * max|o|); L_head and L_proj are then checked
against the norms of the device's own delta recomputed on the host."""
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


def _run(q, K, V, W, keep=None, o_hat=None):
    H, T, d = K.shape
    Lh = torch.empty(H, dtype=torch.float32, device="cuda")
    Lp = torch.empty(H, dtype=torch.float32, device="cuda")
    o = torch.empty((H, d), dtype=torch.float32, device="cuda")
    delta = torch.empty((H, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(L.mikv_perturbation_workspace(H, T, d, W.shape[1]), dtype=torch.uint8, device="cuda")
    L.mikv_output_perturbation(dev(q), dev(K), dev(V), dev(W), Lh, Lp, ws,
                               keep=None if keep is None else dev(np.asarray(keep, np.int32)),
                               o_hat=None if o_hat is None else dev(np.asarray(o_hat, F32)), o=o, delta=delta)
    torch.cuda.synchronize()
    return o.cpu().numpy(), delta.cpu().numpy(), Lh.cpu().numpy(), Lp.cpu().numpy()


def _check(q, K, V, W, keep=None, o_hat=None, what=""):
    o, delta, Lh, Lp = _run(q, K, V, W, keep, o_hat)
    ro, roh, rLh, rLp = O.output_perturbation(q, K, V, W, keep=keep, o_hat=o_hat)
    scale = np.max(np.abs(ro))
    assert np.max(np.abs(o - ro)) <= TOL * scale, f"{what}: o"
    assert np.max(np.abs(delta - (ro - roh))) <= TOL * scale, f"{what}: delta"
    d = K.shape[2]
    dd = delta.astype(F64)
    assert np.allclose(Lh, np.abs(dd).sum(axis=1), rtol=1e-5, atol=1e-30), f"{what}: L_head"
    proj = np.array([np.abs(dd[h] @ W[h * d:(h + 1) * d].astype(F64)).sum() for h in range(K.shape[0])])
    assert np.allclose(Lp, proj, rtol=1e-4, atol=1e-6 * max(1.0, proj.max())), f"{what}: L_proj"
    return Lh, Lp, rLh, rLp


@pytest.mark.parametrize("H,T,d,hidden", [(3, 1, 64, 64), (4, 300, 128, 256), (2, 5000, 64, 100),
                                          (8, 2049, 128, 4096)])
def test_perturbation_random_subsets(H, T, d, hidden):
    print(f"perturbation H={H} T={T} d={d} hidden={hidden}", flush=True)
    rng = np.random.default_rng(H * 1000 + T)
    q = (rng.standard_normal((H, d)) * 1.5).astype(F16)
    K = rng.standard_normal((H, T, d)).astype(F16)
    V = rng.standard_normal((H, T, d)).astype(F16)
    W = (rng.standard_normal((H * d, hidden)) / np.sqrt(hidden)).astype(F16)
    for n_keep in sorted({1, max(1, T // 5), T}):
        keep = np.stack([np.sort(rng.choice(T, n_keep, replace=False)) for _ in range(H)])
        _check(q, K, V, W, keep=keep, what=f"keep {n_keep}")
    ro, _, _, _ = O.output_perturbation(q, K, V, W, keep=[np.arange(T)] * H)
    _check(q, K, V, W, o_hat=ro + rng.standard_normal(ro.shape) * 0.01, what="o_hat")


def test_perturbation_unaligned_w_and_unsorted_keep():
    """W_O at a 2-byte offset (the row-by-row projection path) against the
    16-byte-row path on the same values, and kept indices in any order with
    out-of-range entries (which are ignored) against the sorted set."""
    rng = np.random.default_rng(77)
    H, T, d, hidden = 4, 700, 128, 520
    q = (rng.standard_normal((H, d)) * 1.5).astype(F16)
    K = rng.standard_normal((H, T, d)).astype(F16)
    V = rng.standard_normal((H, T, d)).astype(F16)
    W = (rng.standard_normal((H * d, hidden)) / np.sqrt(hidden)).astype(F16)
    keep = np.stack([np.sort(rng.choice(T, 150, replace=False)) for _ in range(H)])
    Lh, Lp, _, _ = _check(q, K, V, W, keep=keep, what="aligned W")
    # the same W_O one element into a larger buffer: 2-byte aligned
    buf = torch.zeros(H * d * hidden + 1, dtype=torch.float16, device="cuda")
    buf[1:] = torch.from_numpy(W.reshape(-1)).cuda()
    Wu = buf[1:].view(H * d, hidden)
    assert Wu.data_ptr() % 16 != 0
    Lh2 = torch.empty(H, dtype=torch.float32, device="cuda")
    Lp2 = torch.empty(H, dtype=torch.float32, device="cuda")
    ws = torch.empty(L.mikv_perturbation_workspace(H, T, d, hidden), dtype=torch.uint8, device="cuda")
    shuffled = np.stack([np.concatenate([rng.permutation(k), [-3, T, T + 7]]) for k in keep]).astype(np.int32)
    L.mikv_output_perturbation(dev(q), dev(K), dev(V), Wu, Lh2, Lp2, ws, keep=dev(shuffled))
    torch.cuda.synchronize()
    assert np.allclose(Lh2.cpu().numpy(), Lh, rtol=1e-5)
    assert np.allclose(Lp2.cpu().numpy(), Lp, rtol=1e-4)


def test_perturbation_of_selections_h2o_criticalkv_mikv():
    """One Llama-2-shaped layer (8 heads of 128, 2048 prompt tokens, one new
    token, 20% budget): the kept sets of H2O (recent window + heavy hitters
    of the prompt's accumulated attention, the importance set MiKV keeps in
    fp16) and of CriticalKV (the device's two-stage selection on the same
    scores), and MiKV's own output (mikv_decode_attn over the fp16 + INT4
    cache). Each perturbation matches the oracle; the three are reported."""
    cfg = S.CONFIGS["llama2_7b_layer"].scaled(batch=1, hq=8, hkv=8, T=2048)
    hidden = 1024
    q, k, v, _ = S.prefill_tensors(cfg, 1234)
    dims = L.Dims(batch=1, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, group=cfg.G, bits=cfg.bits, cap16=cfg.cap16,
                  capq=cfg.capq())
    acc0 = torch.empty((1, cfg.hkv, cfg.T), dtype=torch.float32, device="cuda")
    ws_s = torch.empty(L.mikv_prefill_scores_workspace(dims, cfg.T), dtype=torch.uint8, device="cuda")
    L.mikv_prefill_scores(dims, cfg.T, dev(q), dev(k), acc0, ws_s)
    b = torch.empty((1, cfg.hkv, cfg.d), dtype=torch.float32, device="cuda")
    ws_b = torch.empty(L.mikv_balance_workspace(dims, cfg.T), dtype=torch.uint8, device="cuda")
    L.mikv_balance_prefill(dims, cfg.T, dev(q), dev(k), b, None, ws_b)
    cache = L.Cache(dims)
    ws_h = torch.empty(L.mikv_h2o_workspace(dims, cfg.T), dtype=torch.uint8, device="cuda")
    L.mikv_h2o_update_select(dims, cache, cfg.T, cfg.recent, cfg.H,
                             src=dict(k=dev(k), v=dev(v), acc0=acc0, b=b), ws=ws_h)
    qd, kd, vd = S.decode_tensors(cfg, 1234, 0)
    o = torch.empty((1, cfg.hq, cfg.d), dtype=torch.float32, device="cuda")
    p16 = torch.empty((1, cfg.hkv, cfg.cap16), dtype=torch.float32, device="cuda")
    ws = torch.zeros(L.mikv_decode_attn_workspace(dims, cfg.T + 1), dtype=torch.uint8, device="cuda")
    L.mikv_decode_attn(dims, cache, cfg.T + 1, dev(qd), dev(kd), dev(vd), b, o, p16, ws)
    torch.cuda.synchronize()
    H, T, B = cfg.hq, cfg.T, cfg.B
    Kf = np.concatenate([k[0], kd[0][:, None]], axis=1)       # [H, T + 1, d], unbalanced fp16
    Vf = np.concatenate([v[0], vd[0][:, None]], axis=1)
    qq = qd[0]
    W = (np.random.default_rng(9).standard_normal((H * cfg.d, hidden)) / np.sqrt(hidden)).astype(F16)
    keep_h2o = np.sort(cache.pos16.cpu().numpy()[0], axis=1)   # B heavy + recent, and the new token T
    assert keep_h2o.shape == (H, B + 1) and np.all(keep_h2o[:, -1] == T)
    idx = torch.empty((H, B), dtype=torch.int32, device="cuda")
    ws_c = torch.empty(L.mikv_criticalkv_workspace(H, T, cfg.d, hidden), dtype=torch.uint8, device="cuda")
    L.mikv_criticalkv_select(acc0[0], dev(v[0]), dev(W), B, 0.5, idx, ws=ws_c)
    keep_ckv = np.concatenate([idx.cpu().numpy(), np.full((H, 1), T)], axis=1)
    res = {}
    res["h2o"] = _check(qq, Kf, Vf, W, keep=keep_h2o, what="h2o")
    res["criticalkv"] = _check(qq, Kf, Vf, W, keep=keep_ckv, what="criticalkv")
    res["mikv"] = _check(qq, Kf, Vf, W, o_hat=o.cpu().numpy()[0], what="mikv")
    for name, (Lh, Lp, _, _) in res.items():
        print(f"  {name}: mean L_proj {Lp.mean():.4g}, mean L_head {Lh.mean():.4g}", flush=True)
    print(f"  heads where CriticalKV < H2O: {(res['criticalkv'][1] < res['h2o'][1]).sum()} of {H}; "
          f"MiKV < H2O: {(res['mikv'][1] < res['h2o'][1]).sum()} of {H}", flush=True)
