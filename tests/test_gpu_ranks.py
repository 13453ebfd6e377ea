"""A stack whose layers have predictors of different ranks (MI355X).

Each layer's predictor rank comes from pi_predictor_ranks (the adaptive predictor of the pages,
PowerInfer methodology and core innovations: per-layer predictors kept small in GPU memory; the
rank follows the entropy of the layer's firing pattern under a budget for all predictor
matrices).  Layers of different firing densities get different ranks; the whole stack then runs
through pi_ffn_layer with ONE workspace sized for the largest rank (the sharing rule of the
header), in both layer orders and as a captured graph, and every layer's result must match the
oracle: mask outside the band, the index list exactly, y within tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from activation_sparse_ffn_rank_amd import DeviceLayer, _abi
from gpu_util import announce, check_mask, check_y, gpu_layer, to_dev

pytestmark = pytest.mark.gpu

D, F = 4096, 8192
DENSITIES = (0.02, 0.05, 0.1, 0.2, 0.35)
R_MIN, R_MAX, R_STEP, R_UNIFORM = 64, 2048, 64, 512


@pytest.fixture(scope="module")
def stack():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = len(DENSITIES)
    probe = [synth.custom_config(D, F, R_MIN, density=dn, seed=700 + i) for i, dn in enumerate(DENSITIES)]
    freqs = [synth.layer_freq(c, 0) for c in probe]
    budget = L * 2 * R_UNIFORM * (D + F)              # the bytes of rank-512 predictors in every layer
    ranks, H = _abi.pi_predictor_ranks([D] * L, [F] * L, freqs, budget, R_MIN, R_MAX, R_STEP)
    assert len(set(int(r) for r in ranks)) >= 3, ranks
    assert all(ranks[i] <= ranks[i + 1] for i in range(L - 1) if H[i] < H[i + 1])
    cfgs = [synth.custom_config(D, F, int(r), density=dn, seed=700 + i)
            for i, (r, dn) in enumerate(zip(ranks, DENSITIES))]
    layers = [synth.make_layer(c, 0) for c in cfgs]
    for lay, fr in zip(layers, freqs):
        assert np.array_equal(lay.freq, fr)
    dls = [DeviceLayer.from_host(lay) for lay in layers]
    announce(f"mixed-rank stack: ranks {list(map(int, ranks))}, entropies {list(H)}")
    return layers, dls


def _shared_ws(dls, B):
    n = max(_abi.pi_workspace_bytes(dl.pred, dl.ffn, B) for dl in dls)
    assert n > 0
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def _check(layer, got, x, what):
    cfg = layer.cfg
    check_mask(got["mask"], oracle.predict(layer.p1, layer.p2, layer.c, x)[0], what)
    idx_ref, n_ref, npred_ref = oracle.compact(got["mask"], layer.slot_of)
    assert np.array_equal(got["idx"], idx_ref) and got["n"] == n_ref and got["n_pred"] == npred_ref, what
    y_ref = oracle.sparse_ffn(cfg.d, cfg.f, cfg.gated, cfg.wtype, layer.w_in, layer.w_down_t, x, idx_ref,
                              b_up=layer.b_up)
    check_y(got["y"], y_ref, cfg.wtype, what)


@pytest.mark.parametrize("B", [1, 4, 16])
def test_mixed_rank_stack_shares_one_workspace(stack, B):
    layers, dls = stack
    ws = _shared_ws(dls, B)
    paths = [_abi.pi_layer_path(dl.pred, dl.ffn, B) for dl in dls]
    order = list(range(len(dls))) + list(reversed(range(len(dls))))
    for step, l in enumerate(order):
        what = f"B={B} step {step} layer {l} rank {layers[l].cfg.r} path {paths[l]}"
        announce(what)
        x = synth.make_x(layers[l].cfg, 0, step, B)
        got = gpu_layer(dls[l], x, ws=ws)
        _check(layers[l], got, x, what)


def test_mixed_rank_stack_graph_replay(stack):
    """The stack captured as one graph over the shared workspace: every replay equals the eager
    pass bit for bit and the oracle within tolerance."""
    layers, dls = stack
    B = 1
    ws = _shared_ws(dls, B)
    L = len(dls)
    xh = [synth.make_x(layers[l].cfg, 0, 100 + l, B) for l in range(L)]
    xs = [to_dev(x) for x in xh]
    ys = [torch.empty((B, D), dtype=torch.float32, device="cuda") for _ in range(L)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for l in range(L):
            _abi.pi_ffn_layer(dls[l].pred, dls[l].ffn, xs[l], B, ys[l], None, None, None, ws)
        torch.cuda.synchronize()
        eager = [y.clone() for y in ys]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for l in range(L):
                _abi.pi_ffn_layer(dls[l].pred, dls[l].ffn, xs[l], B, ys[l], None, None, None, ws)
    for l in range(L):
        got = gpu_layer(dls[l], xh[l], ws=ws)
        assert np.array_equal(got["y"], eager[l].cpu().numpy()), f"layer {l}"
        _check(layers[l], got, xh[l], f"layer {l} eager")
    for rep in range(3):
        announce(f"mixed-rank graph replay {rep}")
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(ys[l], eager[l]), f"replay {rep} layer {l}"
        _abi.pi_ffn_layer(dls[0].pred, dls[0].ffn, xs[0], B, ys[0], None, None, None, ws)   # eager work between
        torch.cuda.synchronize()
    assert _abi.workspace_status(ws) == 0
