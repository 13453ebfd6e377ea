"""pi_sparse_ffn_wide (the sparse FFN at up to 16 tokens on MFMA tiles; fp16 and Q4_0 rows) against
the oracle -- MI355X.

The operation is the method's sparse operator over the listed neurons (PowerInfer, method
section), exactly as pi_sparse_ffn computes it; only the batch range (1..16) and the kernels differ.
Every case compares y element by element with the oracle's fp64 sparse FFN at the same
tolerances, with the rows of unlisted neurons poisoned with NaN (a NaN in y means one was used),
a guard band after y (nothing written past it), a bitwise-repeat check (fixed summation order),
and, at batch <= 8, agreement with pi_sparse_ffn on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from activation_sparse_ffn_rank_amd import DeviceLayer, _abi
from gpu_util import announce, check_y, to_dev

pytestmark = pytest.mark.gpu

F16, Q4 = synth.F16, synth.Q4_0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _abi.lib()


WIDE_CASES = [  # (d, f, gated, wtype, act, B, active share)
    (1024, 4096, False, F16, 0, 16, 0.3), (4096, 3001, True, F16, 0, 16, 0.2), (2048, 2500, False, F16, 1, 16, 0.25),
    (1024, 1000, False, F16, 0, 9, 0.5), (1000, 777, True, F16, 0, 12, 0.4), (768, 2049, False, F16, 0, 13, 1.0),
    (8192, 600, False, F16, 0, 16, 0.2), (4096, 11008, True, F16, 0, 16, 0.1), (1024, 1500, False, F16, 0, 1, 0.1),
    (512, 700, True, F16, 0, 8, 0.3), (2048, 4000, False, F16, 1, 4, 0.2),
    # Q4_0 rows (32-weight blocks with an fp16 scale)
    (1024, 1500, False, Q4, 0, 16, 0.3), (12288, 700, False, Q4, 0, 16, 0.2), (256, 3000, False, Q4, 1, 10, 0.5),
    (2048, 999, False, Q4, 0, 8, 0.15), (768, 400, False, Q4, 0, 1, 1.0),
    # edges: the smallest d_model, d past a 256-column block, a single neuron, an empty list
    (8, 40, False, F16, 0, 16, 0.5), (8, 33, True, F16, 0, 16, 1.0), (264, 100, False, F16, 0, 11, 0.6),
    (256, 1, False, F16, 0, 16, 1.0), (512, 300, False, F16, 0, 16, 0.0), (256, 1, False, Q4, 0, 16, 1.0),
    (512, 300, False, Q4, 0, 16, 0.0),
]


def _layer(d, f, gated, act, seed, wtype=F16):
    cfg = synth.custom_config(d, f, 8, gated=gated, wtype=wtype, bias_up=not gated, seed=seed, act=act)
    w_in, w_dn, b_up, _ = synth.make_ffn(cfg, 0, None, bias_scale=1.0)
    b_down = synth.normal_f16(seed, 0, synth.T_BDOWN, 1, d, 1.0)[0]
    return cfg, w_in, w_dn, b_up, b_down


def _run_wide(dl, x, B, idx, n_listed=None):
    d = dl.ffn.d_model
    guard = 64
    y = torch.full((B * d + guard,), 12345.0, dtype=torch.float32, device="cuda")
    ws = torch.zeros(_abi.pi_sparse_ffn_wide_workspace_bytes(dl.ffn, B), dtype=torch.uint8, device="cuda")
    n = idx.size if n_listed is None else n_listed
    counts = to_dev(np.array([n, n], np.int32))
    idx_d = to_dev(idx) if idx.size else torch.zeros(1, dtype=torch.int32, device="cuda")
    _abi.pi_sparse_ffn_wide(dl.ffn, to_dev(x), B, idx_d, counts, y, ws)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.all(yh[B * d:] == 12345.0), "write past the end of y"
    assert _abi.wide_workspace_status(ws) == 0
    return yh[: B * d].reshape(B, d), (x, idx_d, counts, ws)


@pytest.mark.parametrize("d,f,gated,wtype,act,B,share", WIDE_CASES)
def test_sparse_ffn_wide(d, f, gated, wtype, act, B, share):
    announce(f"sparse_ffn_wide d={d} f={f} gated={gated} wtype={wtype} act={act} B={B} share={share}")
    cfg, w_in, w_dn, b_up, b_down = _layer(d, f, gated, act, seed=d * 5 + f, wtype=wtype)
    rng = np.random.default_rng(d + f + B)
    idx = np.sort(rng.choice(f, int(round(share * f)), replace=False)).astype(np.int32)
    x = synth.normal_f16(cfg.seed, 0, synth.T_X, B, d, 1.0)
    y_ref = oracle.sparse_ffn(d, f, gated, wtype, w_in, w_dn, x, idx, b_up=b_up, b_down=b_down, act=act)
    # poison every row that is not listed (fp16: NaN weights; Q4_0: NaN scales)
    w_in_p, w_dn_p = w_in.copy(), w_dn.copy()
    out = np.setdiff1d(np.arange(f), idx)
    if wtype == F16:
        w_in_p[out] = 0x7E00
        w_dn_p[out] = 0x7E00
    else:
        w_in_p[out, d // 2:] = 0x7E
        w_dn_p[out, d // 2:] = 0x7E
    dl = DeviceLayer(p1=np.zeros((8, d), np.uint16), p2=np.zeros((f, 8), np.uint16), c=np.zeros(f, np.uint16),
                     w_in=w_in_p, w_down_t=w_dn_p, d_model=d, d_ffn=f, gated=gated, wtype=wtype, b_up=b_up,
                     b_down=b_down, act=act)
    y, _ = _run_wide(dl, x, B, idx)
    check_y(y, y_ref, wtype, "sparse_ffn_wide")
    y2, _ = _run_wide(dl, x, B, idx)
    assert np.array_equal(y, y2), "not bitwise repeatable"
    if B <= _abi.PI_MAX_BATCH:
        yv = torch.empty(B * d, dtype=torch.float32, device="cuda")
        ws = torch.zeros(_abi.pi_workspace_bytes(None, dl.ffn, B), dtype=torch.uint8, device="cuda")
        counts = to_dev(np.array([idx.size, idx.size], np.int32))
        idx_d = to_dev(idx) if idx.size else torch.zeros(1, dtype=torch.int32, device="cuda")
        _abi.pi_sparse_ffn(dl.ffn, to_dev(x), B, idx_d, counts, yv, ws)
        torch.cuda.synchronize()
        check_y(y, yv.cpu().numpy().reshape(B, d).astype(np.float64), wtype, "wide vs GEMV form")


def test_sparse_ffn_wide_placement_and_bad_entries():
    """A placement (slot_of) with listed neurons that have no slot, an id past d_ffn and a
    negative id: those entries are skipped, as in pi_sparse_ffn."""
    d, f, B = 2048, 3000, 16
    announce(f"sparse_ffn_wide placement d={d} f={f} B={B}")
    cfg, w_in, w_dn, b_up, b_down = _layer(d, f, False, 0, seed=77)
    rng = np.random.default_rng(3)
    res = np.sort(rng.choice(f, 900, replace=False)).astype(np.int32)
    slot_of = np.full(f, -1, np.int32)
    slot_of[res] = np.arange(res.size, dtype=np.int32)
    listed = np.sort(rng.choice(f, 700, replace=False)).astype(np.int32)
    idx = np.concatenate([listed, np.array([f + 5, -3], np.int32)])
    dl = DeviceLayer(p1=np.zeros((8, d), np.uint16), p2=np.zeros((f, 8), np.uint16), c=np.zeros(f, np.uint16),
                     w_in=w_in[res], w_down_t=w_dn[res], d_model=d, d_ffn=f, gated=False, wtype=F16,
                     slot_of=slot_of, b_up=b_up[res], b_down=b_down)
    x = synth.normal_f16(cfg.seed, 0, synth.T_X, B, d, 1.0)
    y, _ = _run_wide(dl, x, B, idx)
    # n is clamped to n_slots (900): all 702 entries are read, and only resident ids contribute
    kept = np.intersect1d(listed, res)
    y_ref = oracle.sparse_ffn(d, f, False, F16, w_in, w_dn, x, kept, b_up=b_up, b_down=b_down)
    check_y(y, y_ref, F16, "sparse_ffn_wide placement")


def test_sparse_ffn_wide_full_shape_sampled():
    """The 7B-shaped FFN (d 4096, 11008 neurons, ReGLU) at 16 tokens with a 40% union: full y
    against the oracle on four sampled tokens (the oracle's cost grows with the tokens checked)."""
    d, f, B = 4096, 11008, 16
    announce(f"sparse_ffn_wide full shape d={d} f={f} B={B}")
    cfg, w_in, w_dn, _, b_down = _layer(d, f, True, 0, seed=5)
    rng = np.random.default_rng(11)
    idx = np.sort(rng.choice(f, int(0.4 * f), replace=False)).astype(np.int32)
    x = synth.normal_f16(cfg.seed, 0, synth.T_X, B, d, 1.0)
    dl = DeviceLayer(p1=np.zeros((8, d), np.uint16), p2=np.zeros((f, 8), np.uint16), c=np.zeros(f, np.uint16),
                     w_in=w_in, w_down_t=w_dn, d_model=d, d_ffn=f, gated=True, wtype=F16, b_down=b_down)
    y, _ = _run_wide(dl, x, B, idx)
    for b in (0, 5, 10, 15):
        y_ref = oracle.sparse_ffn(d, f, True, F16, w_in, w_dn, x[b:b + 1], idx, b_down=b_down)
        check_y(y[b:b + 1], y_ref, F16, f"full shape token {b}")


def test_sparse_ffn_wide_q4_full_shape_sampled():
    """The 175B-shaped Q4_0 FFN (d 12288, 49152 neurons) at 16 tokens with a 15% union: y against
    the oracle on two sampled tokens."""
    d, f, B = 12288, 49152, 16
    announce(f"sparse_ffn_wide Q4_0 full shape d={d} f={f} B={B}")
    cfg, w_in, w_dn, b_up, b_down = _layer(d, f, False, 0, seed=9, wtype=Q4)
    rng = np.random.default_rng(12)
    idx = np.sort(rng.choice(f, int(0.15 * f), replace=False)).astype(np.int32)
    x = synth.normal_f16(cfg.seed, 0, synth.T_X, B, d, 1.0)
    dl = DeviceLayer(p1=np.zeros((8, d), np.uint16), p2=np.zeros((f, 8), np.uint16), c=np.zeros(f, np.uint16),
                     w_in=w_in, w_down_t=w_dn, d_model=d, d_ffn=f, gated=False, wtype=Q4, b_up=b_up, b_down=b_down)
    y, _ = _run_wide(dl, x, B, idx)
    for b in (3, 14):
        y_ref = oracle.sparse_ffn(d, f, False, Q4, w_in, w_dn, x[b:b + 1], idx, b_up=b_up, b_down=b_down)
        check_y(y[b:b + 1], y_ref, Q4, f"Q4_0 full shape token {b}")


def test_sparse_ffn_wide_rejects():
    d, f = 512, 600
    cfg, w_in, w_dn, b_up, b_down = _layer(d, f, False, 0, seed=1)
    dl = DeviceLayer(p1=np.zeros((8, d), np.uint16), p2=np.zeros((f, 8), np.uint16), c=np.zeros(f, np.uint16),
                     w_in=w_in, w_down_t=w_dn, d_model=d, d_ffn=f, gated=False, wtype=F16, b_up=b_up)
    L = _abi.lib()
    need = _abi.pi_sparse_ffn_wide_workspace_bytes(dl.ffn, 16)
    assert need > 0 and _abi.pi_sparse_ffn_wide_workspace_bytes(dl.ffn, 17) == 0
    assert _abi.pi_sparse_ffn_wide_workspace_bytes(dl.ffn, 0) == 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    x = torch.zeros(16 * d, dtype=torch.int16, device="cuda")
    y = torch.empty(16 * d, dtype=torch.float32, device="cuda")
    idx = torch.zeros(4, dtype=torch.int32, device="cuda")
    counts = torch.zeros(2, dtype=torch.int32, device="cuda")
    import ctypes
    call = lambda B=16, n=need, xp=x.data_ptr(): L.pi_sparse_ffn_wide(ctypes.byref(dl.ffn), xp, B, idx.data_ptr(),
                                                                      counts.data_ptr(), y.data_ptr(), ws.data_ptr(),
                                                                      n, None)
    assert call(B=17) == _abi.PI_ERR_BATCH and call(B=0) == _abi.PI_ERR_BATCH
    assert call(n=need - 1) == _abi.PI_ERR_WORKSPACE
    assert call(xp=None) == _abi.PI_ERR_NULL
    assert call(xp=x.data_ptr() + 2) == _abi.PI_ERR_ALIGN
    assert call() == _abi.PI_OK                                  # empty list: y = b_down (none) = 0
    torch.cuda.synchronize()
    assert torch.all(y == 0).item()


@pytest.mark.parametrize("gated,wtype", [(True, F16), (False, Q4)])
@pytest.mark.parametrize("entry", ["sparse_ffn", "wide"])
def test_h_beyond_fp16_range_is_reported(gated, wtype, entry):
    """The MFMA form carries h as an fp16 pair: one neuron with |h| >= 65504 must set bit 64 of the
    status word (pi_sparse_ffn at batch 3 runs that form for ReGLU and Q4_0 rows; pi_sparse_ffn_wide
    always does), and the same layer without that neuron listed must not."""
    announce(f"h range gated={gated} wtype={wtype} entry={entry}")
    d, f, B, big = 1024, 64, 3, 5
    cfg, w_in, w_dn, b_up, b_down = _layer(d, f, gated, 0, seed=77, wtype=wtype)
    if wtype == F16:
        w_in[big, :d] = 0x5400                    # gate row: 64.0 everywhere -> gate = 65536 at x = 1
        w_in[big, d:] = 0x1400                    # up row: 2^-10 everywhere  -> up = 1
    else:
        w_in[big, : d // 2] = 0xFF                # every code 15: weight 7 * scale
        w_in[big, d // 2:] = np.frombuffer(np.array([0x489A], np.uint16).tobytes() * (d // 32), np.uint8)
    dl = DeviceLayer(p1=np.zeros((8, d), np.uint16), p2=np.zeros((f, 8), np.uint16), c=np.zeros(f, np.uint16),
                     w_in=w_in, w_down_t=w_dn, d_model=d, d_ffn=f, gated=gated, wtype=wtype, b_up=b_up, b_down=b_down)
    x = to_dev(np.full((B, d), 0x3C00, np.uint16))                    # x = 1
    y = torch.empty((B, d), dtype=torch.float32, device="cuda")
    for listed, expect in ((np.array([1, 2, big, 9], np.int32), True), (np.array([1, 2, 9], np.int32), False)):
        counts = to_dev(np.array([listed.size, listed.size], np.int32))
        if entry == "wide":
            ws = torch.zeros(_abi.pi_sparse_ffn_wide_workspace_bytes(dl.ffn, B), dtype=torch.uint8, device="cuda")
            _abi.pi_sparse_ffn_wide(dl.ffn, x, B, to_dev(listed), counts, y, ws)
            torch.cuda.synchronize()
            st = _abi.wide_workspace_status(ws)
        else:
            ws = torch.zeros(_abi.pi_workspace_bytes(None, dl.ffn, B), dtype=torch.uint8, device="cuda")
            assert _abi.pi_sparse_ffn_h_offset(dl.ffn, B)[1] == 3            # the MFMA form runs
            _abi.pi_sparse_ffn(dl.ffn, x, B, to_dev(listed), counts, y, ws)
            torch.cuda.synchronize()
            st = _abi.workspace_status(ws)
        assert bool(st & _abi.PI_STATUS_H_RANGE) == expect, (listed.tolist(), st)


@pytest.mark.parametrize("d,f,gated,wtype,B", [(1024, 900, False, F16, 8), (512, 700, True, F16, 5),
                                                (2048, 600, False, Q4, 16), (264, 333, False, F16, 12)])
def test_h_table_matches_the_listed_rows(d, f, gated, wtype, B):
    """The diagnostic h table of the MFMA form (pi_sparse_ffn_h_offset kind 3, read by
    _abi.sparse_ffn_h) holds, for list position k and token b, the neuron's h: act(W_in x_b + b_up) or
    max(0, W_gate x_b) (W_up x_b), from the rows decoded by the oracle, in fp64."""
    announce(f"h table d={d} f={f} gated={gated} wtype={wtype} B={B}")
    cfg, w_in, w_dn, b_up, b_down = _layer(d, f, gated, 0, seed=900 + d + B, wtype=wtype)
    dl = DeviceLayer(p1=np.zeros((8, d), np.uint16), p2=np.zeros((f, 8), np.uint16), c=np.zeros(f, np.uint16),
                     w_in=w_in, w_down_t=w_dn, d_model=d, d_ffn=f, gated=gated, wtype=wtype, b_up=b_up, b_down=b_down)
    rng = np.random.default_rng(d * 7 + B)
    idx = np.sort(rng.choice(f, size=f // 3, replace=False)).astype(np.int32)
    x = synth.normal_f16(5, 0, synth.T_X, B, d, 1.0)
    ws = torch.zeros(_abi.pi_workspace_bytes(None, dl.ffn, B), dtype=torch.uint8, device="cuda")
    assert _abi.pi_sparse_ffn_h_offset(dl.ffn, B)[1] == 3                # the MFMA form runs
    y = torch.empty((B, d), dtype=torch.float32, device="cuda")
    counts = to_dev(np.array([idx.size, idx.size], np.int32))
    _abi.pi_sparse_ffn(dl.ffn, to_dev(x), B, to_dev(idx), counts, y, ws)
    torch.cuda.synchronize()
    h, ok = _abi.sparse_ffn_h(dl.ffn, B, ws, idx.size)
    h = h.cpu().numpy().astype(np.float64)
    xf = np.array([[oracle.half(int(v)) for v in row] for row in x], np.float64)      # [B][d]
    rb = oracle.row_bytes(wtype, d)
    ref = np.empty((B, idx.size))
    for k, i in enumerate(idx):
        row = w_in[i].view(np.uint8)
        if gated:
            g_ = xf @ oracle.decode_row(row[:rb], wtype, d)
            u_ = xf @ oracle.decode_row(row[rb:2 * rb], wtype, d)
            ref[:, k] = np.maximum(g_, 0.0) * u_
        else:
            u_ = xf @ oracle.decode_row(row[:rb], wtype, d) + oracle.half(int(b_up[i]))
            ref[:, k] = np.maximum(u_, 0.0)
    scale = max(1.0, float(np.abs(ref).max()))
    assert bool(ok.all())
    assert np.abs(h - ref).max() <= 2e-3 * scale, np.abs(h - ref).max()
