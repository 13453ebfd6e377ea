"""Host half of the hybrid split (pi_cold_ffn_host) against the oracle -- runs on the CPU.

The method puts hot neurons on the GPU and computes the cold ones on the CPU, then combines the
partial results (PowerInfer, method section and abstract).  pi_cold_ffn_host computes the
predicted neurons held in host memory; these tests check it against the oracle's sparse FFN over
the same neurons (same tolerances as the device kernels), pin the merge (hot part + cold part =
the whole predicted set), and check its argument handling.  No GPU is needed.
"""
import numpy as np
import pytest

import oracle
import synth
from activation_sparse_ffn_rank_amd import _abi

F16, Q4 = synth.F16, synth.Q4_0


def _layer(d, f, gated, wtype, seed):
    cfg = synth.custom_config(d, f, 8, gated=gated, wtype=wtype, bias_up=not gated, seed=seed)
    w_in, w_dn, b_up, _ = synth.make_ffn(cfg, 0, None, bias_scale=1.0)
    return cfg, w_in, w_dn, b_up


def _split(f, rng, hot_share):
    hot = np.sort(rng.choice(f, int(round(hot_share * f)), replace=False)).astype(np.int32)
    cold = np.setdiff1d(np.arange(f, dtype=np.int32), hot)
    return hot, cold


def _host(cfg, w_in, w_dn, b_up, held):
    """Host descriptor over the rows of neurons `held` (ascending), slot map over all f."""
    slot_of = np.full(cfg.f, -1, np.int32)
    slot_of[held] = np.arange(held.size, dtype=np.int32)
    return _abi.HostFFN(w_in[held], w_dn[held], d_model=cfg.d, d_ffn=cfg.f, gated=cfg.gated, wtype=cfg.wtype,
                        slot_of=slot_of, b_up=None if b_up is None else b_up[held]), slot_of


def _run(host, x, mask, n_threads=0):
    B, d = x.shape
    y = np.full((B, d), np.nan, np.float32)
    ws = np.zeros(_abi.pi_cold_workspace_bytes(host, B), np.uint8)
    n = _abi.pi_cold_ffn_host(host, x, B, mask, y, ws, n_threads)
    return y.astype(np.float64), n


def _check(y, y_ref, wtype):
    err = np.abs(y - y_ref).max(axis=1)
    ref = np.linalg.norm(y_ref, axis=1)
    rel = np.where(ref > 0, np.linalg.norm(y - y_ref, axis=1) / np.maximum(ref, 1e-300), 0.0)
    assert err.max() <= 2e-2, err
    assert rel.max() <= (5e-3 if wtype == F16 else 3e-2), rel


CASES = [  # d, f, gated, wtype, B, predicted share, hot share
    (1024, 4096, False, F16, 1, 0.10, 0.26), (512, 1500, True, F16, 1, 0.2, 0.3), (768, 999, False, F16, 4, 0.3, 0.5),
    (1024, 2048, False, Q4, 1, 0.1, 0.26), (512, 700, False, Q4, 8, 0.2, 0.0), (256, 300, True, F16, 3, 1.0, 0.5),
    (512, 800, False, F16, 16, 0.15, 0.3), (256, 600, False, Q4, 12, 0.2, 0.2),     # up to 16 tokens
]


@pytest.mark.parametrize("d,f,gated,wtype,B,pshare,hshare", CASES)
def test_cold_matches_oracle(d, f, gated, wtype, B, pshare, hshare):
    cfg, w_in, w_dn, b_up = _layer(d, f, gated, wtype, seed=d + f)
    rng = np.random.default_rng(d * 3 + f + B)
    mask = (rng.random(f) < pshare).astype(np.uint8)
    hot, cold = _split(f, rng, hshare)
    host, slot_of = _host(cfg, w_in, w_dn, b_up, cold)
    # poison the host rows of cold neurons that are not predicted: a NaN in y means one was read
    idx = cold[mask[cold] != 0]
    poison = np.setdiff1d(np.arange(cold.size), slot_of[idx])
    wi, wd = host._keep[0], host._keep[1]
    if wtype == F16:
        wi[poison] = 0x7E00
        wd[poison] = 0x7E00
    else:
        wi[poison, d // 2:] = 0x7E
        wd[poison, d // 2:] = 0x7E
    x = synth.normal_f16(cfg.seed, 0, synth.T_X, B, d, 1.0)
    y, n = _run(host, x, mask)
    assert n == idx.size
    y_ref = oracle.sparse_ffn(d, f, gated, wtype, w_in, w_dn, x, idx, b_up=b_up)
    _check(y, y_ref, wtype)


@pytest.mark.parametrize("wtype,B", [(F16, 1), (Q4, 3)])
def test_cold_squared_relu(wtype, B):
    cfg = synth.custom_config(512, 900, 8, gated=False, wtype=wtype, bias_up=True, seed=21, act=1)
    w_in, w_dn, b_up, _ = synth.make_ffn(cfg, 0, None, bias_scale=1.0)
    rng = np.random.default_rng(B)
    mask = (rng.random(cfg.f) < 0.3).astype(np.uint8)
    hot, cold = _split(cfg.f, rng, 0.26)
    slot_of = np.full(cfg.f, -1, np.int32)
    slot_of[cold] = np.arange(cold.size, dtype=np.int32)
    host = _abi.HostFFN(w_in[cold], w_dn[cold], d_model=cfg.d, d_ffn=cfg.f, gated=False, wtype=wtype,
                        slot_of=slot_of, b_up=b_up[cold], act=1)
    x = synth.normal_f16(cfg.seed, 0, synth.T_X, B, cfg.d, 1.0)
    y, n = _run(host, x, mask)
    idx = cold[mask[cold] != 0]
    assert n == idx.size
    _check(y, oracle.sparse_ffn(cfg.d, cfg.f, False, wtype, w_in, w_dn, x, idx, b_up=b_up, act=1), wtype)


def test_hot_plus_cold_is_the_whole_predicted_set():
    """The merge: y(M and H) with b_down + y(M minus H) = y(M) with b_down (the oracle's additivity)."""
    cfg, w_in, w_dn, b_up = _layer(1024, 3000, False, F16, seed=11)
    b_down = synth.normal_f16(cfg.seed, 0, synth.T_BDOWN, 1, cfg.d, 1.0)[0]
    rng = np.random.default_rng(5)
    mask = (rng.random(cfg.f) < 0.15).astype(np.uint8)
    hot, cold = _split(cfg.f, rng, 0.26)
    x = synth.normal_f16(cfg.seed, 0, synth.T_X, 2, cfg.d, 1.0)
    M = np.flatnonzero(mask).astype(np.int32)
    y_hot = oracle.sparse_ffn(cfg.d, cfg.f, False, F16, w_in, w_dn, x, np.intersect1d(M, hot), b_up=b_up,
                              b_down=b_down)
    host, _ = _host(cfg, w_in, w_dn, b_up, cold)
    y_cold, n = _run(host, x, mask)
    assert n == np.intersect1d(M, cold).size
    y_all = oracle.sparse_ffn(cfg.d, cfg.f, False, F16, w_in, w_dn, x, M, b_up=b_up, b_down=b_down)
    _check(y_hot + y_cold, y_all, F16)


def test_result_does_not_depend_on_thread_count():
    cfg, w_in, w_dn, b_up = _layer(2048, 2500, True, F16, seed=3)
    rng = np.random.default_rng(9)
    mask = (rng.random(cfg.f) < 0.3).astype(np.uint8)
    host, _ = _host(cfg, w_in, w_dn, b_up, np.arange(cfg.f, dtype=np.int32))
    x = synth.normal_f16(cfg.seed, 0, synth.T_X, 2, cfg.d, 1.0)
    y1, _ = _run(host, x, mask, n_threads=1)
    y4, _ = _run(host, x, mask, n_threads=4)
    y0, _ = _run(host, x, mask, n_threads=0)
    assert np.array_equal(y1, y4) and np.array_equal(y1, y0)


def test_nothing_predicted_gives_zero():
    cfg, w_in, w_dn, b_up = _layer(512, 600, False, Q4, seed=4)
    host, _ = _host(cfg, w_in, w_dn, b_up, np.arange(cfg.f, dtype=np.int32))
    x = synth.normal_f16(cfg.seed, 0, synth.T_X, 1, cfg.d, 1.0)
    y, n = _run(host, x, np.zeros(cfg.f, np.uint8))
    assert n == 0 and np.all(y == 0.0)


def test_cold_rejects():
    L = _abi.lib()
    import ctypes
    cfg, w_in, w_dn, b_up = _layer(512, 600, False, F16, seed=4)
    host = _abi.HostFFN(w_in, w_dn, d_model=512, d_ffn=600, gated=False, wtype=F16, b_up=b_up)
    x = np.zeros((1, 512), np.uint16)
    m = np.zeros(600, np.uint8)
    y = np.zeros((1, 512), np.float32)
    need = _abi.pi_cold_workspace_bytes(host, 1)
    ws = np.zeros(need, np.uint8)
    call = lambda f=ctypes.byref(host.ffn), B=1, xp=x.ctypes.data, mp=m.ctypes.data, n=need, t=0: \
        L.pi_cold_ffn_host(f, xp, B, mp, y.ctypes.data, None, ws.ctypes.data, n, t)
    assert call() == _abi.PI_OK
    assert call(f=None) == _abi.PI_ERR_NULL
    assert call(xp=None) == _abi.PI_ERR_NULL
    assert call(mp=None) == _abi.PI_ERR_NULL
    assert call(B=0) == _abi.PI_ERR_BATCH and call(B=17) == _abi.PI_ERR_BATCH
    assert call(n=need - 1) == _abi.PI_ERR_WORKSPACE
    assert call(t=-1) == _abi.PI_ERR_SHAPE
    bad = _abi.pi_ffn(512, 600, 0, F16, 600, None, w_in.ctypes.data, w_dn.ctypes.data, None, b_up.ctypes.data)
    assert call(f=ctypes.byref(bad)) == _abi.PI_ERR_DTYPE              # b_down belongs to the device half
    bad = _abi.pi_ffn(500, 600, 0, F16, 600, None, w_in.ctypes.data, w_dn.ctypes.data, None, None)
    assert call(f=ctypes.byref(bad)) == _abi.PI_ERR_SHAPE              # d_model % 8
    assert L.pi_cold_workspace_bytes(ctypes.byref(bad), 1) == 0
    bad = _abi.pi_ffn(512, 600, 0, F16, 600, None, w_in.ctypes.data, w_dn.ctypes.data, None, None, 2)
    assert call(f=ctypes.byref(bad)) == _abi.PI_ERR_DTYPE              # no such activation
    bad = _abi.pi_ffn(512, 600, 1, F16, 600, None, w_in.ctypes.data, w_dn.ctypes.data, None, None, 1)
    assert call(f=ctypes.byref(bad)) == _abi.PI_ERR_DTYPE              # squared ReLU is non-gated
