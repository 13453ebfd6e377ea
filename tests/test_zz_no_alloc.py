"""pi_sparse_ffn_noalloc (the library's own device scratch, no caller workspace) against
pi_sparse_ffn on a caller workspace, through the C ABI: bit-identical y, and within the oracle's
tolerance, on two calls in a row where the second is smaller than the first."""
import numpy as np
import pytest
import torch

import oracle
import synth
from activation_sparse_ffn_rank_amd import DeviceLayer, _abi
from gpu_util import announce, check_y, to_dev

pytestmark = pytest.mark.gpu

F16, Q4 = synth.F16, synth.Q4_0


def _run(d, f, gated, wtype, B, share, seed):
    announce(f"noalloc d={d} f={f} gated={gated} wtype={wtype} B={B} share={share}")
    cfg = synth.custom_config(d, f, 8, gated=gated, wtype=wtype, bias_up=not gated, seed=seed)
    w_in, w_dn, b_up, _ = synth.make_ffn(cfg, 0, None, bias_scale=1.0)
    b_down = synth.normal_f16(seed, 0, synth.T_BDOWN, 1, d, 1.0)[0]
    dl = DeviceLayer(p1=np.zeros((8, d), np.uint16), p2=np.zeros((f, 8), np.uint16), c=np.zeros(f, np.uint16),
                     w_in=w_in, w_down_t=w_dn, d_model=d, d_ffn=f, gated=gated, wtype=wtype, b_up=b_up,
                     b_down=b_down)
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(f, int(round(share * f)), replace=False)).astype(np.int32)
    x = synth.normal_f16(seed, 0, synth.T_X, B, d, 1.0)
    xd, idx_d = to_dev(x), to_dev(idx)
    counts = to_dev(np.array([idx.size, idx.size], np.int32))
    guard = 64
    y_na = torch.full((B * d + guard,), 777.0, dtype=torch.float32, device="cuda")
    y_ws = torch.empty(B * d, dtype=torch.float32, device="cuda")
    ws = torch.zeros(_abi.pi_workspace_bytes(None, dl.ffn, B), dtype=torch.uint8, device="cuda")
    assert ws.numel() <= _abi.PI_NOALLOC_SCRATCH_BYTES
    _abi.pi_sparse_ffn_noalloc(dl.ffn, xd, B, idx_d, counts, y_na)
    _abi.pi_sparse_ffn(dl.ffn, xd, B, idx_d, counts, y_ws, ws)
    torch.cuda.synchronize()
    got = y_na.cpu().numpy()
    assert np.all(got[B * d:] == 777.0), "write past the end of y"
    assert np.array_equal(got[: B * d], y_ws.cpu().numpy()), "noalloc differs from the workspace call"
    y_ref = oracle.sparse_ffn(d, f, gated, wtype, w_in, w_dn, x, idx, b_up=b_up, b_down=b_down)
    check_y(got[: B * d].reshape(B, d), y_ref, wtype, "noalloc")


def test_noalloc_two_calls_second_smaller():
    # the 175B-shaped row width at batch 2 (slab x chunk kernels), then a much smaller layer on
    # the GEMV two-kernel form, on the same scratch
    _run(12288, 4000, False, Q4, 2, 0.3, seed=5)
    _run(1024, 700, True, F16, 1, 0.2, seed=6)


def test_noalloc_every_form():
    # slab x chunk (batch <= 2), GEMV two-kernel (batch 3..5 plain fp16), MFMA (batch >= 6 fp16)
    _run(4096, 3000, True, F16, 1, 0.12, seed=7)
    _run(2048, 2500, False, F16, 4, 0.1, seed=8)
    _run(2048, 1500, False, F16, 8, 0.1, seed=9)
