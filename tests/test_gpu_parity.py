"""GPU parity of every C-ABI entry point against the CPU oracle (MI355X only).

Rules (the method's three decisions are compared on what is unique about them):
* predictor: mask bits equal wherever the oracle's logit is at least 1e-3 from the threshold;
* compaction: index lists and counts bit-exact given the same mask;
* sparse FFN: y per output vector within max-abs 2e-2 and rel-L2 5e-3 (fp16) / 3e-2 (Q4_0),
  given the same index list.
Unit cases use scale-1 biases and a nonzero b_down so that every term is large enough to
break the tolerance if it were dropped.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from activation_sparse_ffn_rank_amd import DeviceLayer, _abi
from gpu_util import (LAYER_ENTRIES, LOGIT_ATOL, announce, check_layer_against_oracle, check_mask, check_y, gpu_layer,
                      gpu_predict, to_dev)

pytestmark = pytest.mark.gpu

F16, Q4 = synth.F16, synth.Q4_0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _abi.lib()


# ----------------------------------------------------------------------------- predictor

PRED_CASES = [  # (d, f, r, B) -- ragged f, tiny and maximal rank, every batch width class
    (256, 1000, 8, 1), (1024, 4096, 128, 1), (512, 4099, 520, 3), (4096, 11008, 1024, 1),
    (1024, 2500, 2048, 2), (12288, 3001, 1024, 8), (8192, 777, 1024, 5),
    # past 8 tokens: the first matrix in two passes, the second on MFMA (z as an fp16 pair)
    (1024, 4096, 128, 9), (4096, 11008, 1024, 16), (512, 4099, 520, 13), (1024, 2500, 2048, 16),
    (12288, 3001, 1024, 12), (256, 1000, 8, 16),
]


@pytest.mark.parametrize("d,f,r,B", PRED_CASES)
def test_predict(d, f, r, B):
    announce(f"predict d={d} f={f} r={r} B={B}")
    cfg = synth.custom_config(d, f, r, density=0.1, seed=d + f + r)
    p1, p2, c, _ = synth.make_predictor(cfg, 0)
    # predictor-only case: the FFN part of the layer is a placeholder that is never used
    dl = DeviceLayer(p1=p1, p2=p2, c=c, w_in=np.zeros((f, 8), np.uint16), w_down_t=np.zeros((f, 8), np.uint16),
                     d_model=8, d_ffn=f, gated=False, wtype=F16)
    x = synth.make_x(cfg, 0, 0, B)
    logits, mask = gpu_predict(dl, x)
    ref, _, _ = oracle.predict(p1, p2, c, x)
    assert np.abs(logits - ref).max() < LOGIT_ATOL
    check_mask(mask, ref, "predict")
    assert np.array_equal(mask, (logits > 0).any(axis=0).astype(np.uint8))   # GPU mask follows GPU logits


# ----------------------------------------------------------------------------- compaction

@pytest.mark.parametrize("f", [1, 63, 64, 4095, 4096, 4097, 11008, 49152])
@pytest.mark.parametrize("density", [0.0, 0.05, 0.5, 1.0])
def test_compact(f, density):
    announce(f"compact f={f} density={density}")
    rng = np.random.default_rng(f + int(density * 100))
    mask = (rng.random(f) < density).astype(np.uint8)
    mask[mask == 1] = rng.integers(1, 256, int(mask.sum()))      # any nonzero byte means "predicted"
    slot_of = np.where(rng.random(f) < 0.26, np.arange(f), -1).astype(np.int32)
    for so in (None, slot_of):
        idx = torch.full((f,), -7, dtype=torch.int32, device="cuda")
        counts = torch.full((2,), -7, dtype=torch.int32, device="cuda")
        _abi.pi_compact(to_dev(mask), f, None if so is None else to_dev(so), idx, counts)
        torch.cuda.synchronize()
        ref, n, npred = oracle.compact((mask != 0).astype(np.uint8), so)
        got = counts.cpu().numpy()
        assert got.tolist() == [n, npred]
        assert np.array_equal(idx[:n].cpu().numpy(), ref)
        assert np.all(idx[n:].cpu().numpy() == -7)               # nothing written past n


# ----------------------------------------------------------------------------- sparse FFN

FFN_CASES = [  # (d, f, gated, wtype, B, active share)
    (1024, 4096, False, F16, 1, 0.1), (1024, 1000, True, F16, 1, 0.3), (4096, 3001, True, F16, 2, 0.05),
    (768, 2049, False, F16, 3, 1.0), (512, 700, False, Q4, 1, 0.2), (1024, 1500, False, Q4, 4, 0.1),
    (2048, 999, False, Q4, 8, 0.15), (1024, 800, True, F16, 8, 0.2), (12288, 1200, False, Q4, 8, 0.1),
    (8192, 600, False, F16, 5, 0.2), (256, 64, False, F16, 1, 0.0), (7168, 513, False, F16, 4, 0.5),
    # gated with x in column chunks; every neuron listed over several passes of the up kernel
    (8192, 301, True, F16, 6, 0.3), (256, 12000, False, Q4, 3, 0.8),
    # edges of the batch > 2 form: the smallest d_model, a single neuron, an empty list
    (8, 40, False, F16, 3, 0.5), (8, 33, True, F16, 8, 1.0), (256, 1, False, Q4, 4, 1.0), (512, 300, False, Q4, 5, 0.0),
    # batch <= 2 (one launch of slab x chunk workgroups): ragged last slab, chunks that take several
    # rounds, both batch widths for every row kind, the 7B- and 175B-shaped row widths
    (1280, 20000, False, Q4, 2, 0.5), (2056, 5000, True, F16, 2, 0.6), (1032, 9000, False, F16, 1, 0.7),
    (2048, 3000, False, Q4, 1, 1.0), (1024, 2000, False, F16, 2, 0.3), (8, 50, False, F16, 1, 0.5),
    (4096, 11008, True, F16, 1, 0.12), (12288, 6000, False, Q4, 1, 0.4), (12288, 3000, False, Q4, 2, 0.2),
]


def _ffn_layer(d, f, gated, wtype, seed):
    cfg = synth.custom_config(d, f, 8, gated=gated, wtype=wtype, bias_up=not gated, seed=seed)
    w_in, w_dn, b_up, _ = synth.make_ffn(cfg, 0, None, bias_scale=1.0)
    b_down = synth.normal_f16(seed, 0, synth.T_BDOWN, 1, d, 1.0)[0]
    return cfg, w_in, w_dn, b_up, b_down


@pytest.mark.parametrize("d,f,gated,wtype,B,share", FFN_CASES)
def test_sparse_ffn(d, f, gated, wtype, B, share):
    announce(f"sparse_ffn d={d} f={f} gated={gated} wtype={wtype} B={B} share={share}")
    cfg, w_in, w_dn, b_up, b_down = _ffn_layer(d, f, gated, wtype, seed=d * 7 + f)
    rng = np.random.default_rng(d + f + B)
    idx = np.sort(rng.choice(f, int(round(share * f)), replace=False)).astype(np.int32)
    x = synth.normal_f16(cfg.seed, 0, synth.T_X, B, d, 1.0)
    y_ref = oracle.sparse_ffn(d, f, gated, wtype, w_in, w_dn, x, idx, b_up=b_up, b_down=b_down)
    # poison every row that is not listed: a NaN in y means an inactive row was read
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
                     b_down=b_down)
    guard = 64
    y = torch.full((B * d + guard,), 12345.0, dtype=torch.float32, device="cuda")
    ws = torch.zeros(_abi.pi_workspace_bytes(None, dl.ffn, B), dtype=torch.uint8, device="cuda")
    counts = to_dev(np.array([idx.size, idx.size], np.int32))
    idx_d = to_dev(idx) if idx.size else torch.zeros(1, dtype=torch.int32, device="cuda")
    _abi.pi_sparse_ffn(dl.ffn, to_dev(x), B, idx_d, counts, y, ws)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.all(yh[B * d:] == 12345.0), "write past the end of y"
    check_y(yh[: B * d].reshape(B, d), y_ref, wtype, "sparse_ffn")
    # bitwise repeatable (deterministic reduction)
    y2 = torch.empty(B * d, dtype=torch.float32, device="cuda")
    _abi.pi_sparse_ffn(dl.ffn, to_dev(x), B, idx_d, counts, y2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy(), yh[: B * d])
    # every form keeps the status word at its fixed offset: 0 after two good calls
    assert _abi.workspace_status(ws) == 0


@pytest.mark.parametrize("d,f,wtype,B", [(1024, 3000, F16, 1), (1024, 3000, F16, 2), (2048, 999, Q4, 1),
                                         (768, 2049, F16, 5), (12288, 700, Q4, 8)])
def test_sparse_ffn_squared_relu(d, f, wtype, B):
    """Squared ReLU h = max(0, W_up x + b_up)^2 through the persistent form (batch <= 2) and the
    two-kernel form (batch > 2, or x in LDS column chunks)."""
    announce(f"sparse_ffn squared ReLU d={d} f={f} wtype={wtype} B={B}")
    cfg, w_in, w_dn, b_up, b_down = _ffn_layer(d, f, False, wtype, seed=d + 5 * f)
    rng = np.random.default_rng(d + f + B)
    idx = np.sort(rng.choice(f, f // 4, replace=False)).astype(np.int32)
    x = synth.normal_f16(cfg.seed, 0, synth.T_X, B, d, 1.0)
    y_ref = oracle.sparse_ffn(d, f, False, wtype, w_in, w_dn, x, idx, b_up=b_up, b_down=b_down, act=1)
    dl = DeviceLayer(p1=np.zeros((8, d), np.uint16), p2=np.zeros((f, 8), np.uint16), c=np.zeros(f, np.uint16),
                     w_in=w_in, w_down_t=w_dn, d_model=d, d_ffn=f, gated=False, wtype=wtype, b_up=b_up,
                     b_down=b_down, act=1)
    y = torch.empty((B, d), dtype=torch.float32, device="cuda")
    ws = torch.zeros(_abi.pi_workspace_bytes(None, dl.ffn, B), dtype=torch.uint8, device="cuda")
    _abi.pi_sparse_ffn(dl.ffn, to_dev(x), B, to_dev(idx), to_dev(np.array([idx.size, idx.size], np.int32)), y, ws)
    torch.cuda.synchronize()
    assert _abi.workspace_status(ws) == 0
    check_y(y.cpu().numpy(), y_ref, wtype, "sparse_ffn squared ReLU")


def test_sparse_ffn_skips_bad_index_entries():
    """Out-of-range ids or non-resident slots are skipped, and counts beyond n_slots are clamped."""
    d, f = 512, 300
    cfg, w_in, w_dn, b_up, b_down = _ffn_layer(d, f, False, F16, seed=3)
    x = synth.normal_f16(3, 0, synth.T_X, 1, d, 1.0)
    idx = np.array([5, -1, 17, 100000, 42], np.int32)
    dl = DeviceLayer(p1=np.zeros((8, d), np.uint16), p2=np.zeros((f, 8), np.uint16), c=np.zeros(f, np.uint16),
                     w_in=w_in, w_down_t=w_dn, d_model=d, d_ffn=f, gated=False, wtype=F16, b_up=b_up, b_down=b_down)
    ws = torch.zeros(_abi.pi_workspace_bytes(None, dl.ffn, 1), dtype=torch.uint8, device="cuda")
    y = torch.empty(d, dtype=torch.float32, device="cuda")
    _abi.pi_sparse_ffn(dl.ffn, to_dev(x), 1, to_dev(idx), to_dev(np.array([5, 5], np.int32)), y, ws)
    torch.cuda.synchronize()
    y_ref = oracle.sparse_ffn(d, f, False, F16, w_in, w_dn, x, np.array([5, 17, 42], np.int32), b_up=b_up,
                              b_down=b_down)
    check_y(y.cpu().numpy()[None], y_ref, F16, "bad-entries")


# ----------------------------------------------------------------------------- whole layer

LAYER_CASES = [  # small layers spanning several tiles, ragged f, placement, all FFN kinds
    dict(d=1024, f=4096, r=128, gated=False, wtype=F16, bias_up=True, density=0.1),
    dict(d=2048, f=5503, r=256, gated=True, wtype=F16, bias_up=False, density=0.12),
    dict(d=1536, f=6001, r=512, gated=False, wtype=F16, bias_up=True, density=0.06, hot_frac=0.26),
    dict(d=2048, f=4100, r=1024, gated=False, wtype=Q4, bias_up=True, density=0.05),
    # squared ReLU: the tail kernel (small f) and separate kernels (large f), fp16 and Q4_0
    dict(d=1024, f=4096, r=128, gated=False, wtype=F16, bias_up=True, density=0.1, act=1),
    dict(d=1024, f=40000, r=128, gated=False, wtype=Q4, bias_up=True, density=0.05, act=1),
    # separate kernels at every batch (too many neurons for the tail kernel): placement, ReGLU
    dict(d=1024, f=40000, r=128, gated=False, wtype=F16, bias_up=True, density=0.05, hot_frac=0.26),
    dict(d=1024, f=33000, r=256, gated=True, wtype=F16, bias_up=False, density=0.06),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=["relu", "reglu", "placement", "q4_0", "squared_relu",
                                                  "squared_relu_q4_0_large_f", "placement_large_f",
                                                  "reglu_large_f"])
@pytest.mark.parametrize("B", [1, 4, 8, 12, 16])
def test_ffn_layer(case, B):
    announce(f"ffn_layer {case} B={B}")
    cfg = synth.custom_config(**case, seed=B * 100 + case["d"])
    layer = synth.make_layer(cfg, 0, bias_scale=1.0, b_down=True)
    dl = DeviceLayer.from_host(layer)
    for t in range(3):
        x = synth.make_x(cfg, 0, t, B)
        check_layer_against_oracle(layer, dl, x, f"layer t={t}")


def test_layer_relu_1024x4096_all_tokens():
    """The single-layer 1024x4096 rank-128 configuration, all 64 seeded tokens at batch 1."""
    cfg = synth.CONFIGS[1]
    announce("config relu-ffn-1x1024x4096, 64 tokens")
    layer = synth.make_layer(cfg, 0)
    dl = DeviceLayer.from_host(layer)
    ws = dl.workspace(1)
    dens = []
    for t in range(cfg.tokens):
        x = synth.make_x(cfg, 0, t, 1)
        r = check_layer_against_oracle(layer, dl, x, f"t={t}")
        dens.append(r["n"] / cfg.f)
    assert abs(np.mean(dens) - cfg.density) < 0.25 * cfg.density
    del ws


def test_empty_prediction_gives_down_bias():
    """No neuron fires (all offsets very negative): y = b_down exactly, nothing else is read."""
    cfg = synth.custom_config(1024, 2000, 64, seed=77)
    layer = synth.make_layer(cfg, 0, b_down=True)
    layer.c[:] = np.float16(-60000.0).view(np.uint16)
    dl = DeviceLayer.from_host(layer)
    got = gpu_layer(dl, synth.make_x(cfg, 0, 0, 2))
    assert got["n"] == 0 and got["n_pred"] == 0 and got["mask"].sum() == 0
    bd = layer.b_down.view(np.float16).astype(np.float32)
    assert np.array_equal(got["y"], np.tile(bd, (2, 1)))


def test_every_neuron_fires_equals_dense():
    """All offsets very positive: every neuron is listed and y is the dense MLP."""
    cfg = synth.custom_config(1024, 3000, 64, seed=78)
    layer = synth.make_layer(cfg, 0, bias_scale=1.0, b_down=True)
    layer.c[:] = np.float16(60000.0).view(np.uint16)
    dl = DeviceLayer.from_host(layer)
    x = synth.make_x(cfg, 0, 0, 3)
    got = gpu_layer(dl, x)
    assert got["n"] == cfg.f and np.array_equal(got["idx"], np.arange(cfg.f))
    y_dense, _ = oracle.dense_ffn(cfg.d, cfg.f, False, F16, layer.w_in, layer.w_down_t, x, b_up=layer.b_up,
                                  b_down=layer.b_down)
    check_y(got["y"], y_dense, F16, "dense")


def test_layer_is_deterministic():
    cfg = synth.custom_config(4096, 11008, 1024, gated=True, bias_up=False, density=0.12, seed=5)
    layer = synth.make_layer(cfg, 0)
    dl = DeviceLayer.from_host(layer)
    x = synth.make_x(cfg, 0, 0, 1)
    a, b = gpu_layer(dl, x), gpu_layer(dl, x)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["idx"], b["idx"])


@pytest.mark.parametrize("entry", ["layer", "two_step"])
def test_graph_replay_matches_eager(entry):
    """The launch sequence captured into a HIP graph (as the benchmark runs it) gives, on every
    replay, exactly what eager calls give."""
    run = LAYER_ENTRIES[entry]
    cfg = synth.custom_config(2048, 5000, 256, gated=False, bias_up=True, density=0.1, seed=9, layers=3)
    layers = [synth.make_layer(cfg, l) for l in range(3)]
    dls = [DeviceLayer.from_host(L) for L in layers]
    xs = [to_dev(synth.make_x(cfg, l, 0, 1)) for l in range(3)]
    ws = dls[0].workspace(1)
    ys = [torch.empty((1, cfg.d), dtype=torch.float32, device="cuda") for _ in range(3)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for l in range(3):
            run(dls[l].pred, dls[l].ffn, xs[l], 1, ys[l], None, None, None, ws)
        torch.cuda.synchronize()
        eager = [y.clone() for y in ys]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for l in range(3):
                run(dls[l].pred, dls[l].ffn, xs[l], 1, ys[l], None, None, None, ws)
    # the eager result of each layer against the oracle, given the GPU's own list (same launches)
    refs = []
    for l in range(3):
        x = synth.make_x(cfg, l, 0, 1)
        got = gpu_layer(dls[l], x)
        assert np.array_equal(got["y"], eager[l].cpu().numpy()), f"layer {l}: outputs depend on the requested lists"
        check_mask(got["mask"], oracle.predict(layers[l].p1, layers[l].p2, layers[l].c, x)[0], f"layer {l}")
        refs.append(oracle.sparse_ffn(cfg.d, cfg.f, False, cfg.wtype, layers[l].w_in, layers[l].w_down_t, x,
                                      got["idx"], b_up=layers[l].b_up))
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for l in range(3):
            assert torch.equal(ys[l], eager[l]), f"replay {rep} layer {l}"
            check_y(ys[l].cpu().numpy(), refs[l], cfg.wtype, f"replay {rep} layer {l} vs oracle")
        # eager work between replays
        run(dls[0].pred, dls[0].ffn, xs[0], 1, ys[0], None, None, None, ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("entry", ["layer", "two_step"])
def test_layer_outputs_are_optional(entry):
    """mask/idx/counts outputs change nothing about y (bitwise)."""
    run = LAYER_ENTRIES[entry]
    cfg = synth.custom_config(2048, 6000, 512, gated=True, bias_up=False, density=0.1, seed=31)
    layer = synth.make_layer(cfg, 0)
    dl = DeviceLayer.from_host(layer)
    x = to_dev(synth.make_x(cfg, 0, 0, 2))
    ws = dl.workspace(2)
    y1 = torch.empty((2, cfg.d), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y1)
    run(dl.pred, dl.ffn, x, 2, y1, None, None, None, ws)
    got = gpu_layer(dl, synth.make_x(cfg, 0, 0, 2), ws=ws, entry=entry)
    run(dl.pred, dl.ffn, x, 2, y2, None, None, None, ws)
    torch.cuda.synchronize()
    assert _abi.workspace_status(ws) == 0
    assert torch.equal(y1, y2) and np.array_equal(y1.cpu().numpy(), got["y"])


@pytest.mark.parametrize("entry", ["layer", "two_step"])
def test_many_calls_share_one_workspace(entry):
    """Back-to-back launches on one workspace (epochs advance, counters reset) stay exact."""
    run = LAYER_ENTRIES[entry]
    cfg = synth.custom_config(1024, 4096, 128, density=0.1, seed=41, layers=2)
    layers = [synth.make_layer(cfg, l) for l in range(2)]
    dls = [DeviceLayer.from_host(L) for L in layers]
    ws = dls[0].workspace(1)
    xs = [to_dev(synth.make_x(cfg, l, t, 1)) for t in range(5) for l in range(2)]
    ref = []
    for i, x in enumerate(xs):
        y = torch.empty((1, cfg.d), dtype=torch.float32, device="cuda")
        run(dls[i % 2].pred, dls[i % 2].ffn, x, 1, y, None, None, None, ws)
        ref.append(y)
    torch.cuda.synchronize()
    for rep in range(3):
        for i, x in enumerate(xs):
            y = torch.empty((1, cfg.d), dtype=torch.float32, device="cuda")
            run(dls[i % 2].pred, dls[i % 2].ffn, x, 1, y, None, None, None, ws)
            torch.cuda.synchronize()
            assert torch.equal(y, ref[i]), (rep, i)
    assert _abi.workspace_status(ws) == 0
    got = check_layer_against_oracle(layers[1], dls[1], synth.make_x(cfg, 1, 4, 1), "after many calls", entries=(entry,))
    assert got["n"] > 0


@pytest.mark.parametrize("case", [
    dict(d=1024, f=4096, r=128, gated=False, wtype=F16, bias_up=True, density=0.1),          # tail kernel
    dict(d=2048, f=5503, r=256, gated=True, wtype=F16, bias_up=False, density=0.12),         # tail kernel, ReGLU
    dict(d=1024, f=40000, r=128, gated=False, wtype=F16, bias_up=True, density=0.05),        # separate kernels
    dict(d=1024, f=40000, r=128, gated=False, wtype=Q4, bias_up=True, density=0.05),         # ... Q4_0
    dict(d=1536, f=6001, r=512, gated=False, wtype=F16, bias_up=True, density=0.06, hot_frac=0.26),
], ids=["tail_relu", "tail_reglu", "split_relu", "split_q4_0", "tail_placement"])
@pytest.mark.parametrize("B", [1, 2])
def test_layer_reads_no_unlisted_row(case, B):
    """pi_ffn_layer reads no row outside the predicted, resident set: with every other row poisoned
    with NaN (fp16 weights, or Q4_0 scales) y is bitwise the unpoisoned y and matches the oracle, and
    nothing is written past y (guard band)."""
    announce(f"poisoned layer {case} B={B}")
    cfg = synth.custom_config(**case, seed=300 + B)
    layer = synth.make_layer(cfg, 0, bias_scale=1.0, b_down=True)
    dl = DeviceLayer.from_host(layer)
    x = synth.make_x(cfg, 0, 0, B)
    clean = gpu_layer(dl, x)
    listed = clean["idx"]
    assert clean["n"] > 0
    slots = listed if layer.slot_of is None else layer.slot_of[listed]
    keep = np.zeros(layer.w_in.shape[0], bool)
    keep[slots] = True
    w_in_p, w_dn_p = layer.w_in.copy(), layer.w_down_t.copy()
    if cfg.wtype == F16:
        w_in_p[~keep] = 0x7E00
        w_dn_p[~keep] = 0x7E00
    else:
        w_in_p[~keep, cfg.d // 2:] = 0x7E
        w_dn_p[~keep, cfg.d // 2:] = 0x7E
    dlp = DeviceLayer(p1=layer.p1, p2=layer.p2, c=layer.c, w_in=w_in_p, w_down_t=w_dn_p, d_model=cfg.d, d_ffn=cfg.f,
                      gated=cfg.gated, wtype=cfg.wtype, slot_of=layer.slot_of, b_up=layer.b_up, b_down=layer.b_down)
    guard = 64
    y = torch.full((B * cfg.d + guard,), 4242.0, dtype=torch.float32, device="cuda")
    ws = dlp.workspace(B)
    _abi.pi_ffn_layer(dlp.pred, dlp.ffn, to_dev(x), B, y, None, None, None, ws)
    torch.cuda.synchronize()
    assert _abi.workspace_status(ws) == 0
    yh = y.cpu().numpy()
    assert np.all(yh[B * cfg.d:] == 4242.0), "write past the end of y"
    assert np.array_equal(yh[: B * cfg.d].reshape(B, cfg.d), clean["y"]), "an unlisted row changed y"
    y_ref = oracle.sparse_ffn(cfg.d, cfg.f, cfg.gated, cfg.wtype, layer.w_in, layer.w_down_t, x, listed,
                              b_up=layer.b_up, b_down=layer.b_down, slot_of=layer.slot_of)
    check_y(yh[: B * cfg.d].reshape(B, cfg.d), y_ref, cfg.wtype, "poisoned layer")


def test_split_layer_matches_whole_layer():
    """pi_predict_hidden + pi_ffn_layer_from_hidden is bitwise pi_ffn_layer, and z = ReLU(P1 x) >= 0."""
    for case in (dict(d=2048, f=5503, r=256, gated=True, wtype=F16, bias_up=False, density=0.12),
                 dict(d=1536, f=6001, r=512, gated=False, wtype=F16, bias_up=True, density=0.06, hot_frac=0.26),
                 dict(d=2048, f=4100, r=1024, gated=False, wtype=Q4, bias_up=True, density=0.05)):
        cfg = synth.custom_config(**case, seed=71)
        layer = synth.make_layer(cfg, 0, bias_scale=1.0, b_down=True)
        dl = DeviceLayer.from_host(layer)
        for B in (1, 3):
            announce(f"split layer {case} B={B}")
            x = synth.make_x(cfg, 0, 1, B)
            whole = gpu_layer(dl, x, entry="layer")
            split = gpu_layer(dl, x, entry="two_step")
            assert np.array_equal(whole["y"], split["y"]) and np.array_equal(whole["idx"], split["idx"])
            z = torch.empty((B, cfg.r), dtype=torch.float32, device="cuda")
            _abi.pi_predict_hidden(dl.pred, to_dev(x), B, z)
            torch.cuda.synchronize()
            assert bool((z >= 0).all()) and bool(torch.isfinite(z).all())
            check_layer_against_oracle(layer, dl, x, f"split B={B}", entries=("two_step",))
