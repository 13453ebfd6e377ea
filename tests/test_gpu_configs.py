"""Parity at the full layer shapes of the five measured stacks (MI355X only).

Each case generates full-size layers -- the first and the last layer of the stack and three more
drawn with a seeded generator (they all have different hot sets and weights) -- runs pi_ffn_layer,
the entry point the benchmark replays, on several seeded tokens (or token batches) per layer, and
checks it against the oracle by the end-to-end rule: masks agree outside the 1e-3 logit band, the
index list is bit-exact given the GPU's mask, and y agrees within the stated tolerances given that
list.  The batch variants use the union of the per-token masks.  The single small layer runs all
64 of its tokens in test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import synth
from activation_sparse_ffn_rank_amd import DeviceLayer, _abi
from gpu_util import announce, check_layer_against_oracle

pytestmark = pytest.mark.gpu

CASES = [(2, 1), (2, 16), (3, 1), (3, 4), (4, 1), (5, 1), (5, 8), (5, 16)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _abi.lib()


def layers_of(cfg):
    """First, last and three seeded random layers of the stack (fewer when the stack is short)."""
    rng = np.random.default_rng(1000 + cfg.cid)
    picks = {0, cfg.layers - 1}
    if cfg.layers > 2:
        picks |= set(int(v) for v in rng.choice(np.arange(1, cfg.layers - 1), size=min(3, cfg.layers - 2),
                                                 replace=False))
    return sorted(picks)


@pytest.mark.parametrize("cid,B", CASES)
def test_full_size_layers(cid, B):
    cfg = synth.CONFIGS[cid]
    shares, dens = [], []
    steps = 8 if B == 1 else 4
    for l in layers_of(cfg):
        announce(f"config {cid} ({cfg.name}) layer {l} B={B}, {steps} steps")
        layer = synth.make_layer(cfg, l)
        dl = DeviceLayer.from_host(layer)
        for t in range(steps):
            x = synth.make_x(cfg, l, t, B)
            r = check_layer_against_oracle(layer, dl, x, f"config {cid} layer {l} token {t} B={B}")
            shares.append(r["n"] / max(r["n_pred"], 1))
            dens.append(r["n_pred"] / cfg.f)
        del dl, layer
        torch.cuda.empty_cache()
    if cfg.hot_frac is None:
        assert all(s == 1.0 for s in shares)
    else:
        assert 0.5 < float(np.mean(shares)) < 1.0           # hottest 26% cover most firings
    if B == 1:
        assert 0.4 * cfg.density < float(np.mean(dens)) < 2.5 * cfg.density
