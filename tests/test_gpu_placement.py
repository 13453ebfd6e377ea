"""Budgeted placement driving the device (MI355X + host cores).

pi_place chooses, under a device-memory budget, which neurons of each layer of a small mixed stack
(fp16 ReLU, Q4_0 ReLU and fp16 ReGLU layers: different neuron sizes and firing laws, so the budget
is not split evenly) are resident on the GPU (PowerInfer, method section: an offline policy over
activation frequency and bandwidth picks the GPU-resident neurons; README: the result is the GPU
index, sized by a VRAM budget).  Each layer then runs on the device over its resident rows
(pi_ffn_layer with pi_place's slot_of) and on the host over the rest (pi_cold_ffn_host), and the
sum must equal the oracle's sparse FFN over every predicted neuron of the device's mask.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from activation_sparse_ffn_rank_amd import DeviceLayer, _abi
from gpu_util import announce, check_mask, check_y, to_dev

pytestmark = pytest.mark.gpu

STACK = [  # (d, f, r, gated, wtype, bias_up, density)
    (1024, 8192, 256, False, synth.F16, True, 0.08),
    (1024, 8192, 256, False, synth.Q4_0, True, 0.05),
    (1024, 6000, 256, True, synth.F16, False, 0.12),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _abi.lib()


def test_pi_place_slot_of_drives_the_hybrid_layer():
    cfgs = [synth.custom_config(d, f, r, gated=g, wtype=w, bias_up=b, density=dn, seed=600 + i)
            for i, (d, f, r, g, w, b, dn) in enumerate(STACK)]
    nbytes = [(3 if c.gated else 2) * c.row_bytes() for c in cfgs]
    freqs = [synth.layer_freq(c, 0) for c in cfgs]
    total = sum(c.f * nb for c, nb in zip(cfgs, nbytes))
    budget = int(0.3 * total)
    slot_ofs, n_placed, t_exp = _abi.pi_place([c.f for c in cfgs], nbytes, freqs, budget, 8e12, 1e11)
    assert sum(int(n) * nb for n, nb in zip(n_placed, nbytes)) <= budget
    assert len(set(int(n) / c.f for n, c in zip(n_placed, cfgs))) > 1       # the budget is not split evenly
    for i, (cfg, so, npl) in enumerate(zip(cfgs, slot_ofs, n_placed)):
        hot = np.flatnonzero(so >= 0).astype(np.int32)
        assert hot.size == int(npl) and np.array_equal(so[hot], np.arange(hot.size))   # ascending-id slots
        layer = synth.make_layer(cfg, 0, hot=hot)
        assert np.array_equal(layer.slot_of, so)
        dl = DeviceLayer.from_host(layer)
        cold = np.setdiff1d(np.arange(cfg.f, dtype=np.int32), hot)
        w_in_c, w_dn_c, b_up_c, _ = synth.make_ffn(cfg, 0, cold)
        slot_c = np.full(cfg.f, -1, np.int32)
        slot_c[cold] = np.arange(cold.size, dtype=np.int32)
        host = _abi.HostFFN(w_in_c, w_dn_c, d_model=cfg.d, d_ffn=cfg.f, gated=cfg.gated, wtype=cfg.wtype,
                            slot_of=slot_c, b_up=b_up_c)
        w_in_all, w_dn_all, b_up_all, _ = synth.make_ffn(cfg, 0, None)
        covered, predicted = 0, 0
        for B in (1, 4):
            announce(f"placed layer {i} ({hot.size} of {cfg.f} resident) B={B}")
            ws_h = np.zeros(_abi.pi_cold_workspace_bytes(host, B), np.uint8)
            x = synth.make_x(cfg, 0, B, B)
            y = torch.empty((B, cfg.d), dtype=torch.float32, device="cuda")
            mask = torch.empty(cfg.f, dtype=torch.uint8, device="cuda")
            counts = torch.empty(2, dtype=torch.int32, device="cuda")
            ws = dl.workspace(B)
            _abi.pi_ffn_layer(dl.pred, dl.ffn, to_dev(x), B, y, mask, None, counts, ws)
            torch.cuda.synchronize()
            assert _abi.workspace_status(ws) == 0
            m = mask.cpu().numpy()
            check_mask(m, oracle.predict(layer.p1, layer.p2, layer.c, x)[0], f"layer {i} B={B}")
            y_cold = np.empty((B, cfg.d), np.float32)
            n_cold = _abi.pi_cold_ffn_host(host, x, B, m, y_cold, ws_h)
            M = np.flatnonzero(m).astype(np.int32)
            n, n_pred = (int(v) for v in counts.cpu().numpy())
            assert n_pred == M.size and n == np.intersect1d(M, hot).size and n + n_cold == M.size
            covered, predicted = covered + n, predicted + n_pred
            y_ref = oracle.sparse_ffn(cfg.d, cfg.f, cfg.gated, cfg.wtype, w_in_all, w_dn_all, x, M, b_up=b_up_all)
            check_y(y.cpu().numpy().astype(np.float64) + y_cold, y_ref, cfg.wtype, f"layer {i} B={B}")
        # the most frequent neurons are the ones kept, so the device covers more than its share of rows
        assert covered / predicted > hot.size / cfg.f
        del dl
