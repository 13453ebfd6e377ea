"""The hybrid split end to end on the placement stack's full layer shape (MI355X + host cores).

The device runs the whole layer over the resident (hottest 26%) neurons and returns the union mask;
the host computes the predicted neurons that are not resident (pi_cold_ffn_host, over the cold
rows in host memory); the sum must match the oracle's sparse FFN over every predicted neuron
(PowerInfer, method section: hot neurons on the GPU, cold ones on the CPU, partial results merged).
The mask itself is checked against the oracle's logits outside the 1e-3 band, and the oracle then
runs on the device's mask.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from activation_sparse_ffn_rank_amd import DeviceLayer, _abi
from gpu_util import announce, check_mask, check_y

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _abi.lib()


def test_hot_on_device_plus_cold_on_host_is_the_whole_layer():
    cfg = synth.CONFIGS[4]
    l = 0
    announce(f"hybrid config 4 ({cfg.name}) layer {l}")
    layer = synth.make_layer(cfg, l)
    dl = DeviceLayer.from_host(layer)
    cold = np.setdiff1d(np.arange(cfg.f, dtype=np.int32), layer.hot)
    w_in_c, w_dn_c, b_up_c, _ = synth.make_ffn(cfg, l, cold)
    slot_c = np.full(cfg.f, -1, np.int32)
    slot_c[cold] = np.arange(cold.size, dtype=np.int32)
    host = _abi.HostFFN(w_in_c, w_dn_c, d_model=cfg.d, d_ffn=cfg.f, gated=cfg.gated, wtype=cfg.wtype,
                        slot_of=slot_c, b_up=b_up_c)
    ws_h = np.zeros(_abi.pi_cold_workspace_bytes(host, 1), np.uint8)
    w_in_all, w_dn_all, b_up_all, _ = synth.make_ffn(cfg, l, None)
    for t in range(2):
        x = synth.make_x(cfg, l, t, 1)
        y = torch.empty((1, cfg.d), dtype=torch.float32, device="cuda")
        mask = torch.empty(cfg.f, dtype=torch.uint8, device="cuda")
        ws = dl.workspace(1)
        _abi.pi_ffn_layer(dl.pred, dl.ffn, torch.from_numpy(x.view(np.int16)).cuda(), 1, y, mask, None, None, ws)
        torch.cuda.synchronize()
        assert _abi.workspace_status(ws) == 0
        m = mask.cpu().numpy()
        logits, _, _ = oracle.predict(layer.p1, layer.p2, layer.c, x)
        check_mask(m, logits, f"token {t}")
        y_cold = np.empty((1, cfg.d), np.float32)
        n_cold = _abi.pi_cold_ffn_host(host, x, 1, m, y_cold, ws_h)
        M = np.flatnonzero(m).astype(np.int32)
        assert n_cold == np.intersect1d(M, cold).size and n_cold > 0
        y_ref = oracle.sparse_ffn(cfg.d, cfg.f, cfg.gated, cfg.wtype, w_in_all, w_dn_all, x, M, b_up=b_up_all)
        check_y(y.cpu().numpy().astype(np.float64) + y_cold, y_ref, cfg.wtype, f"hybrid token {t}")
