"""Shared helpers of the GPU parity tests (no test functions here)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from activation_sparse_ffn_rank_amd import DeviceLayer, _abi

BAND = 1e-3                  # predictor logits closer than this to 0 may flip either way
MAX_ABS = 2e-2               # per output vector
REL_L2 = {synth.F16: 5e-3, synth.Q4_0: 3e-2}
LOGIT_ATOL = 1e-3            # |l_gpu - l_oracle|; fp32 accumulation error is ~1e-5 here


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, wtype: int, what: str = "") -> dict:
    """Spec tolerances per output vector: max-abs <= 2e-2 and rel-L2 <= 5e-3 (fp16) / 3e-2 (Q4_0)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    assert y_gpu.shape == y_ref.shape, what
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    worst = dict(max_abs=0.0, rel_l2=0.0)
    for b in range(y_ref.shape[0]):
        diff = y_gpu[b] - y_ref[b]
        mx = float(np.abs(diff).max()) if diff.size else 0.0
        nrm = float(np.linalg.norm(y_ref[b]))
        rel = float(np.linalg.norm(diff) / nrm) if nrm > 0 else 0.0
        assert mx <= MAX_ABS, f"{what} b={b}: max-abs {mx:.3e}"
        if nrm > 0:
            assert rel <= REL_L2[wtype], f"{what} b={b}: rel-L2 {rel:.3e}"
        worst["max_abs"] = max(worst["max_abs"], mx)
        worst["rel_l2"] = max(worst["rel_l2"], rel)
    return worst


def check_mask(mask_gpu: np.ndarray, logits_ref: np.ndarray, what: str = "") -> int:
    """Union-mask bits must match wherever the oracle's logits are decided outside the band."""
    must1 = (logits_ref >= BAND).any(axis=0)
    must0 = (logits_ref <= -BAND).all(axis=0)
    m = mask_gpu.astype(bool)
    assert m[must1].all(), f"{what}: {int((~m[must1]).sum())} neurons predicted by the oracle are missing"
    assert not m[must0].any(), f"{what}: {int(m[must0].sum())} neurons fire on the GPU only"
    assert set(np.unique(mask_gpu)) <= {0, 1}
    return int((~must1 & ~must0).sum())          # don't-care neurons


def gpu_predict(dl: DeviceLayer, x: np.ndarray):
    B = x.shape[0]
    xd = to_dev(x)
    mask = torch.empty(dl.d_ffn, dtype=torch.uint8, device="cuda")
    logits = torch.empty((B, dl.d_ffn), dtype=torch.float32, device="cuda")
    ws = torch.empty(_abi.pi_workspace_bytes(dl.pred, None, B), dtype=torch.uint8, device="cuda")
    _abi.pi_predict(dl.pred, xd, B, mask, logits, ws)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), mask.cpu().numpy()


def _layer_two_step(pred, ffn, x, batch, y, mask_out, idx_out, counts_out, ws, stream=None):
    """pi_ffn_layer as its two published steps: pi_predict_hidden, then pi_ffn_layer_from_hidden."""
    z = torch.empty((batch, pred.rank), dtype=torch.float32, device="cuda")
    _abi.pi_predict_hidden(pred, x, batch, z, stream)
    _abi.pi_ffn_layer_from_hidden(pred, ffn, x, batch, z, y, mask_out, idx_out, counts_out, ws, stream)


LAYER_ENTRIES = {"layer": _abi.pi_ffn_layer, "two_step": _layer_two_step}


def gpu_layer(dl: DeviceLayer, x: np.ndarray, ws: torch.Tensor | None = None, entry: str = "layer"):
    B = x.shape[0]
    xd = to_dev(x)
    y = torch.empty((B, dl.d_model), dtype=torch.float32, device="cuda")
    mask = torch.empty(dl.d_ffn, dtype=torch.uint8, device="cuda")
    idx = torch.empty(dl.d_ffn, dtype=torch.int32, device="cuda")
    counts = torch.empty(2, dtype=torch.int32, device="cuda")
    ws = dl.workspace(B) if ws is None else ws
    LAYER_ENTRIES[entry](dl.pred, dl.ffn, xd, B, y, mask, idx, counts, ws)
    torch.cuda.synchronize()
    assert _abi.workspace_status(ws) == 0, "a cross-workgroup wait timed out"
    n = int(counts[0])
    return dict(y=y.cpu().numpy(), mask=mask.cpu().numpy(), idx=idx[:n].cpu().numpy(), n=n,
                n_pred=int(counts[1]))


def check_layer_against_oracle(layer, dl: DeviceLayer, x: np.ndarray, what: str, b_down=None,
                               entries=("layer",)) -> dict:
    """End-to-end rule: masks agree outside the band; given the GPU's mask the oracle's index list
    is identical; given that list the oracle's y agrees within tolerance.  Checked for every
    layer entry point named in `entries` that takes this shape."""
    cfg = layer.cfg
    B = x.shape[0]
    logits_ref, _, _ = oracle.predict(layer.p1, layer.p2, layer.c, x)
    bd = layer.b_down if b_down is None else b_down
    worst = None
    for entry in entries:
        tag = f"{what} [{entry}]"
        got = gpu_layer(dl, x, entry=entry)
        dont_care = check_mask(got["mask"], logits_ref, tag)
        idx_ref, n_ref, npred_ref = oracle.compact(got["mask"], layer.slot_of)
        assert np.array_equal(got["idx"], idx_ref) and got["n"] == n_ref and got["n_pred"] == npred_ref, tag
        y_ref = oracle.sparse_ffn(cfg.d, cfg.f, cfg.gated, cfg.wtype, layer.w_in, layer.w_down_t, x, idx_ref,
                                  b_up=layer.b_up, b_down=bd, slot_of=layer.slot_of, act=cfg.act)
        w = check_y(got["y"], y_ref, cfg.wtype, tag)
        w.update(n=got["n"], n_pred=got["n_pred"], dont_care=dont_care)
        if worst is None:
            worst = w
    return worst
