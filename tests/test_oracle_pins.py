"""Pins of the CPU oracle to facts fixed outside it (CPU only, no GPU).

Each test checks the oracle against something it cannot agree with by construction: the
IEEE binary16 definition (through numpy's conversion), hand-worked fixtures in
tests/golden/, closed forms (zero predictor weights, all-zero Q4_0 codes), a library matmul
of the plain dense MLP, brute force over every mask of a tiny layer with exact integer
arithmetic, and the invariants of the method itself -- computing only the neurons that fire
gives the dense result, neurons left out contribute exactly nothing, and disjoint neuron
sets add up (PowerInfer, arXiv 2312.12456: hot/cold split of neurons whose partial results
are merged, and neuron-aware operators that skip inactive neurons).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import synth

F16, Q4 = oracle.F16, oracle.Q4_0


def h16(a):
    """float -> fp16 bit patterns (exact for the small dyadic values the fixtures use)."""
    arr = np.asarray(a, dtype=np.float64)
    out = arr.astype(np.float16)
    assert np.array_equal(out.astype(np.float64), arr), "fixture value not exact in fp16"
    return out.view(np.uint16)


@pytest.fixture(scope="module")
def golden(golden_dir):
    with open(os.path.join(golden_dir, "tiny_layers.json")) as fh:
        return json.load(fh)


# ----------------------------------------------------------------------------- binary16

def test_half_exhaustive_matches_ieee_binary16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_row(bits, F16, 65536)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # spot values from the format definition
    assert oracle.half(0x3C00) == 1.0 and oracle.half(0xC000) == -2.0
    assert oracle.half(0x0001) == 2.0 ** -24 and oracle.half(0x7BFF) == 65504.0
    assert oracle.half(0x7C00) == np.inf


# ----------------------------------------------------------------------------- Q4_0

def pack_q4(codes, scales):
    """Rows of Q4_0 bytes from integer codes: weight 2j -> low nibble of byte j."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, d = codes.shape
    lo, hi = codes[:, 0::2], codes[:, 1::2]
    body = (lo | (hi << 4)).astype(np.uint8)
    sc = h16(scales).reshape(n, d // 32).view(np.uint8)
    return np.concatenate([body, sc], axis=1)


def test_q4_0_decode_golden(golden):
    g = golden["q4_0"]
    rows = pack_q4(g["W_up_codes"], np.asarray(g["W_up_scale"]).reshape(2, 1))
    assert rows[0, 0] == 0x4A and rows[0, 15] == 0xF8
    assert oracle.row_bytes(Q4, 32) == rows.shape[1] == 18
    w = oracle.decode_row(rows[0], Q4, 32)
    assert list(w[:2]) == g["w_up_row0_first"] and w[31] == g["w_up_row0_last"]
    assert np.all(w[2:31] == 0.0)


def test_q4_0_code_eight_is_zero_and_scale_per_block():
    d = 96
    codes = np.full((1, d), 8, dtype=np.uint8)
    codes[0, 32] = 9                     # first weight of block 1
    codes[0, 95] = 0                     # last weight of block 2
    rows = pack_q4(codes, np.array([[3.0, 0.5, 0.125]]))
    w = oracle.decode_row(rows[0], Q4, d)
    expect = np.zeros(d)
    expect[32] = 0.5
    expect[95] = 0.125 * -8
    assert np.array_equal(w, expect)


# ----------------------------------------------------------------------------- predictor

def test_predictor_golden_rank1(golden):
    g = golden["predictor_rank1"]
    for case in g["cases"]:
        logits, mask, _ = oracle.predict(h16(g["P1"]), h16(g["P2"]), h16(g["c"]), h16([case["x"]]))
        assert list(logits[0]) == case["logits"]
        assert list(mask) == case["mask"]


def test_predictor_golden_relu_layer(golden):
    g = golden["relu"]
    for case in g["cases"]:
        logits, mask, tok = oracle.predict(h16(g["P1"]), h16(g["P2"]), h16(g["c"]), h16(case["x"]),
                                           want_tok_masks=True)
        assert logits.tolist() == case["logits"]
        assert tok.tolist() == case["token_masks"]
        assert mask.tolist() == case["mask"]


def test_predictor_zero_p2_gives_offsets():
    rng = np.random.default_rng(0)
    d, f, r = 64, 200, 8
    p1 = h16(rng.integers(-4, 5, (r, d)) / 8)
    p2 = np.zeros((f, r), dtype=np.uint16)
    c = h16(rng.integers(-8, 9, f) / 4)
    x = h16(rng.integers(-8, 9, (3, d)) / 4)
    logits, mask, _ = oracle.predict(p1, p2, c, x)
    cv = c.view(np.float16).astype(np.float64)
    assert np.array_equal(logits, np.tile(cv, (3, 1)))
    assert np.array_equal(mask, (cv > 0).astype(np.uint8))
    # c = 0 with P2 = 0: every logit is exactly zero and nothing fires (strict threshold)
    logits, mask, _ = oracle.predict(p1, p2, np.zeros(f, np.uint16), x)
    assert np.all(logits == 0.0) and mask.sum() == 0


def test_predictor_matches_library_matmul_and_union():
    cfg = synth.custom_config(256, 300, 32, seed=7)
    p1, p2, c, _ = synth.make_predictor(cfg, 0)
    x = np.stack([synth.make_x(cfg, 0, t, 1)[0] for t in range(4)])
    logits, mask, tok = oracle.predict(p1, p2, c, x, want_tok_masks=True)
    P1 = p1.view(np.float16).astype(np.float64)
    P2 = p2.view(np.float16).astype(np.float64)
    X = x.view(np.float16).astype(np.float64)
    ref = np.maximum(X @ P1.T, 0.0) @ P2.T + c.view(np.float16).astype(np.float64)
    np.testing.assert_allclose(logits, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(tok, (logits > 0).astype(np.uint8))
    assert np.array_equal(mask, tok.max(axis=0))
    # a batch row is computed exactly as that token alone
    for b in range(4):
        lb, mb, _ = oracle.predict(p1, p2, c, x[b:b + 1])
        assert np.array_equal(lb[0], logits[b]) and np.array_equal(mb, tok[b])


# ----------------------------------------------------------------------------- compaction

@pytest.mark.parametrize("f", [1, 7, 64, 1000, 4099])
@pytest.mark.parametrize("density", [0.0, 0.03, 0.5, 1.0])
def test_compact_brute_force(f, density):
    rng = np.random.default_rng(f)
    mask = (rng.random(f) < density).astype(np.uint8)
    idx, n, n_pred = oracle.compact(mask)
    assert np.array_equal(idx, np.flatnonzero(mask)) and n == n_pred == int(mask.sum())
    slot_of = np.where(rng.random(f) < 0.3, np.arange(f), -1).astype(np.int32)
    idx, n, n_pred = oracle.compact(mask, slot_of)
    assert np.array_equal(idx, np.flatnonzero(mask.astype(bool) & (slot_of >= 0)))
    assert n_pred == int(mask.sum()) and n == idx.size


# ----------------------------------------------------------------------------- sparse FFN

def test_relu_golden(golden):
    g = golden["relu"]
    d, f = g["d"], g["f"]
    w_in, wd, bu, bd = h16(g["W_up"]), h16(g["W_down_t"]), h16(g["b_up"]), h16(g["b_down"])
    for case in g["cases"]:
        x = h16(case["x"])
        y, h = oracle.sparse_ffn(d, f, False, F16, w_in, wd, x, case["idx"], b_up=bu, b_down=bd, want_h=True)
        assert y.tolist() == case["y"] and h.tolist() == case["h"]
        res = oracle.ffn_layer(_golden_layer(g), x)
        assert res["mask"].tolist() == case["mask"] and res["idx"].tolist() == case["idx"]
        assert (res["n"], res["n_pred"]) == (case["n"], case["n_pred"])
        assert res["y"].tolist() == case["y"]
        if "y_dense" in case:
            yd, tm = oracle.dense_ffn(d, f, False, F16, w_in, wd, x, b_up=bu, b_down=bd)
            assert yd.tolist() == case["y_dense"] and tm.tolist() == case["true_mask"]
    pl = g["placement"]
    slot_of = np.asarray(pl["slot_of"], dtype=np.int32)
    resident = np.flatnonzero(slot_of >= 0)
    layer = _golden_layer(g, slot_of=slot_of, rows=resident)
    res = oracle.ffn_layer(layer, h16(pl["x"]))
    assert res["idx"].tolist() == pl["idx"] and (res["n"], res["n_pred"]) == (pl["n"], pl["n_pred"])
    assert res["y"].tolist() == pl["y"]


def _golden_layer(g, slot_of=None, rows=None):
    cfg = synth.custom_config(g["d"], g["f"], g["r"], bias_up=True)
    sel = slice(None) if rows is None else rows
    return synth.Layer(cfg, 0, h16(g["P1"]), h16(g["P2"]), h16(g["c"]), np.zeros(g["f"]), slot_of, rows,
                       h16(g["W_up"])[sel], h16(g["W_down_t"])[sel], h16(g["b_up"])[sel], h16(g["b_down"]))


def test_reglu_golden(golden):
    g = golden["reglu"]
    d, f = g["d"], g["f"]
    w_in = np.concatenate([h16(g["W_gate"]), h16(g["W_up"])], axis=1)     # gate row, then up row
    wd, bd, x = h16(g["W_down_t"]), h16(g["b_down"]), h16(g["x"])
    y, h = oracle.sparse_ffn(d, f, True, F16, w_in, wd, x, g["idx"], b_down=bd, want_h=True)
    assert y.tolist() == g["y"] and h.tolist() == g["h"]
    yd, tm = oracle.dense_ffn(d, f, True, F16, w_in, wd, x, b_down=bd)
    assert yd.tolist() == g["y_dense"] and tm.tolist() == g["true_mask"]


def test_q4_0_ffn_golden(golden):
    g = golden["q4_0"]
    d, f = g["d"], g["f"]
    w_in = pack_q4(g["W_up_codes"], np.asarray(g["W_up_scale"]).reshape(f, 1))
    wd = pack_q4(g["W_down_codes"], np.asarray(g["W_down_scale"]).reshape(f, 1))
    x = np.zeros((1, d))
    x[0, :2] = g["x_first"]
    x[0, 31] = g["x_last"]
    y, h = oracle.sparse_ffn(d, f, False, Q4, w_in, wd, h16(x), g["idx"], b_up=h16(g["b_up"]), want_h=True)
    assert h.tolist() == g["h"] and np.all(y == g["y_value"])


def test_q4_0_zero_codes_give_relu_bias():
    d, f = 64, 5
    codes = np.full((f, d), 8, dtype=np.uint8)
    w = pack_q4(codes, np.ones((f, 2)))
    bu = h16([-1.0, 0.5, 2.0, 0.0, 3.0])
    bd = h16(np.arange(d) / 16)
    x = h16(np.random.default_rng(1).integers(-4, 4, (2, d)) / 4)
    y, h = oracle.sparse_ffn(d, f, False, Q4, w, w, x, np.arange(f), b_up=bu, b_down=bd, want_h=True)
    assert np.array_equal(h, np.tile([0.0, 0.5, 2.0, 0.0, 3.0], (2, 1)))
    assert np.array_equal(y, np.tile(np.arange(d) / 16, (2, 1)))


def _tiny_int_layer(rng, d, f, gated):
    """Integer-valued fp16 weights: every product and sum below is an exact integer."""
    g = rng.integers(-3, 4, (f, d))
    u = rng.integers(-3, 4, (f, d))
    wd = rng.integers(-3, 4, (f, d))
    bu = rng.integers(-4, 5, f)
    bd = rng.integers(-4, 5, d)
    x = rng.integers(-3, 4, (2, d))
    return g, u, wd, bu, bd, x


@pytest.mark.parametrize("gated", [False, True])
def test_brute_force_all_masks_tiny(gated):
    """d=8, f=10: every one of the 2^10 neuron sets against an exact integer triple loop."""
    rng = np.random.default_rng(5 + gated)
    d, f = 8, 10
    g, u, wd, bu, bd, x = _tiny_int_layer(rng, d, f, gated)
    w_in = np.concatenate([h16(g), h16(u)], axis=1) if gated else h16(u)
    bias = None if gated else h16(bu)
    for bits in range(1 << f):
        idx = [i for i in range(f) if bits >> i & 1]
        y = oracle.sparse_ffn(d, f, gated, F16, w_in, h16(wd), h16(x), np.asarray(idx, np.int32),
                              b_up=bias, b_down=h16(bd))
        for b in range(2):
            expect = [int(v) for v in bd]
            for i in idx:
                if gated:
                    gv = sum(int(g[i, t]) * int(x[b, t]) for t in range(d))
                    uv = sum(int(u[i, t]) * int(x[b, t]) for t in range(d))
                    hv = max(gv, 0) * uv
                else:
                    hv = max(sum(int(u[i, t]) * int(x[b, t]) for t in range(d)) + int(bu[i]), 0)
                for j in range(d):
                    expect[j] += hv * int(wd[i, j])
            assert y[b].tolist() == expect, (bits, b)


def _np_decode(rows, wtype, d):
    if wtype == F16:
        return rows.view(np.float16).astype(np.float64).reshape(rows.shape[0], -1)
    codes = rows[:, : d // 2]
    lo, hi = (codes & 15).astype(np.float64), (codes >> 4).astype(np.float64)
    q = np.empty((rows.shape[0], d))
    q[:, 0::2], q[:, 1::2] = lo, hi
    sc = rows[:, d // 2:].copy().view(np.float16).astype(np.float64)
    return (q - 8.0) * np.repeat(sc, 32, axis=1)


def _numpy_dense(layer, x):
    """The plain MLP with a library matmul: h = act(W x), y = h W_down^T (all neurons)."""
    cfg = layer.cfg
    d = cfg.d
    X = x.view(np.float16).astype(np.float64)
    if cfg.gated:
        win = layer.w_in.reshape(layer.n_slots, 2, -1)
        G = _np_decode(np.ascontiguousarray(win[:, 0]), cfg.wtype, d)
        U = _np_decode(np.ascontiguousarray(win[:, 1]), cfg.wtype, d)
        H = np.maximum(X @ G.T, 0.0) * (X @ U.T)
    else:
        U = _np_decode(layer.w_in, cfg.wtype, d)
        pre = X @ U.T
        if layer.b_up is not None:
            pre = pre + layer.b_up.view(np.float16).astype(np.float64)
        H = np.maximum(pre, 0.0)
        if getattr(cfg, "act", 0):
            H = H * H                                   # squared ReLU
    Y = H @ _np_decode(layer.w_down_t, cfg.wtype, d)
    if layer.b_down is not None:
        Y = Y + layer.b_down.view(np.float16).astype(np.float64)
    return Y, H


LAYER_CASES = [
    dict(d=256, f=700, r=32, gated=False, wtype=F16, bias_up=True),
    dict(d=256, f=513, r=32, gated=True, wtype=F16, bias_up=False),
    dict(d=320, f=300, r=16, gated=False, wtype=Q4, bias_up=True),
    dict(d=256, f=400, r=32, gated=False, wtype=F16, bias_up=True, act=1),
    dict(d=256, f=300, r=16, gated=False, wtype=Q4, bias_up=True, act=1),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=["relu", "reglu", "q4_0", "squared_relu", "squared_relu_q4_0"])
def test_dense_equals_sparse_invariants(case):
    """I1 (all neurons = dense MLP), I2 (true mask = dense, bit-exact), I3 (NaN rows outside
    the set change nothing), I4 (disjoint sets add), I8 (batch rows equal single tokens)."""
    cfg = synth.custom_config(**case, density=0.2, seed=11)
    layer = synth.make_layer(cfg, 0, bias_scale=1.0, b_down=True)
    d, f = cfg.d, cfg.f
    x = np.concatenate([synth.make_x(cfg, 0, t, 1) for t in range(3)])
    yref, H = _numpy_dense(layer, x)
    args = (d, f, cfg.gated, cfg.wtype, layer.w_in, layer.w_down_t)
    kw = dict(b_up=layer.b_up, b_down=layer.b_down, act=cfg.act)
    # I1
    y_all = oracle.sparse_ffn(*args, x, np.arange(f), **kw)
    np.testing.assert_allclose(y_all, yref, rtol=1e-10, atol=1e-10)
    y_dense, tm = oracle.dense_ffn(*args, x, **kw)
    assert np.array_equal(y_dense, y_all)
    assert np.array_equal(tm.astype(bool), H != 0)
    for b in range(3):
        true_idx = np.flatnonzero(tm[b])
        # I2: only the truly active neurons, bit-exact with dense
        yb = oracle.sparse_ffn(*args, x[b:b + 1], true_idx, **kw)
        assert np.array_equal(yb[0], y_dense[b])
        # I8: the batch row equals the token computed alone
        assert np.array_equal(oracle.sparse_ffn(*args, x[b:b + 1], np.arange(f), **kw)[0], y_all[b])
    # I3: poison every row outside a random set with NaN
    rng = np.random.default_rng(3)
    sel = np.sort(rng.choice(f, f // 5, replace=False)).astype(np.int32)
    y_sel = oracle.sparse_ffn(*args, x, sel, **kw)
    out = np.setdiff1d(np.arange(f), sel)
    w_in_p, wd_p = layer.w_in.copy(), layer.w_down_t.copy()
    if cfg.wtype == F16:
        w_in_p[out] = 0x7E00
        wd_p[out] = 0x7E00
    else:
        w_in_p[out, cfg.d // 2:] = 0x7E        # NaN scale bytes (0x7E7E is a NaN)
        wd_p[out, cfg.d // 2:] = 0x7E
    y_poison = oracle.sparse_ffn(d, f, cfg.gated, cfg.wtype, w_in_p, wd_p, x, sel, **kw)
    assert np.array_equal(y_poison, y_sel)
    # I4: y(A) + y(B) - b_down = y(A u B) for disjoint A, B
    a, bset = sel[::2], sel[1::2]
    ya = oracle.sparse_ffn(*args, x, a, **kw)
    yb = oracle.sparse_ffn(*args, x, bset, **kw)
    bdv = layer.b_down.view(np.float16).astype(np.float64)
    np.testing.assert_allclose(ya + yb - bdv, y_sel, rtol=1e-10, atol=1e-10)


def test_placement_slots_are_an_indirection():
    """Resident rows addressed through slot_of give what the full matrix gives for them."""
    cfg = synth.custom_config(256, 600, 32, density=0.15, hot_frac=0.3, seed=21)
    layer = synth.make_layer(cfg, 0, bias_scale=1.0)
    full_in, full_dn, full_bu, _ = synth.make_ffn(cfg, 0, None, bias_scale=1.0)
    x = synth.make_x(cfg, 0, 0, 2)
    res = oracle.ffn_layer(layer, x)
    assert np.array_equal(full_in[layer.hot], layer.w_in)
    expect_idx = np.flatnonzero(res["mask"].astype(bool) & (layer.slot_of >= 0))
    assert np.array_equal(res["idx"], expect_idx) and res["n_pred"] == int(res["mask"].sum())
    y_full = oracle.sparse_ffn(cfg.d, cfg.f, False, F16, full_in, full_dn, x, res["idx"], b_up=full_bu)
    assert np.array_equal(res["y"], y_full)
    # and the cold remainder completes the layer (hot/cold split merges by addition)
    cold = np.setdiff1d(np.flatnonzero(res["mask"]), res["idx"]).astype(np.int32)
    y_cold = oracle.sparse_ffn(cfg.d, cfg.f, False, F16, full_in, full_dn, x, cold, b_up=full_bu)
    y_union = oracle.sparse_ffn(cfg.d, cfg.f, False, F16, full_in, full_dn, x, np.flatnonzero(res["mask"]),
                                b_up=full_bu)
    np.testing.assert_allclose(res["y"] + y_cold, y_union, rtol=1e-10, atol=1e-10)


def test_empty_active_set_gives_down_bias():
    cfg = synth.custom_config(128, 64, 8, seed=2)
    layer = synth.make_layer(cfg, 0, b_down=True)
    x = synth.make_x(cfg, 0, 0, 3)
    y = oracle.sparse_ffn(cfg.d, cfg.f, False, F16, layer.w_in, layer.w_down_t, x, np.zeros(0, np.int32),
                          b_up=layer.b_up, b_down=layer.b_down)
    assert np.array_equal(y, np.tile(layer.b_down.view(np.float16).astype(np.float64), (3, 1)))
    y0 = oracle.sparse_ffn(cfg.d, cfg.f, False, F16, layer.w_in, layer.w_down_t, x, np.zeros(0, np.int32))
    assert np.all(y0 == 0.0)


def test_thread_count_does_not_change_results():
    cfg = synth.custom_config(512, 900, 64, gated=True, bias_up=False, seed=9)
    layer = synth.make_layer(cfg, 0)
    x = synth.make_x(cfg, 0, 0, 2)
    n0 = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        a = oracle.ffn_layer(layer, x)
        oracle.set_num_threads(max(2, n0))
        b = oracle.ffn_layer(layer, x)
    finally:
        oracle.set_num_threads(n0)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["logits"], b["logits"])


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.sparse_ffn(100, 10, False, Q4, np.zeros((10, 57), np.uint8), np.zeros((10, 57), np.uint8),
                          np.zeros((1, 100), np.uint16), np.arange(3))      # Q4_0 needs d % 32 == 0
    with pytest.raises(ValueError):
        oracle.sparse_ffn(32, 10, False, F16, np.zeros((4, 32), np.uint16), np.zeros((4, 32), np.uint16),
                          np.zeros((1, 32), np.uint16), np.array([5], np.int32))   # slot 5 >= n_slots


def test_squared_relu_by_hand():
    """Squared ReLU (README FAQ lists it beside ReLU and ReGLU), one neuron worked by hand, every
    value exact in fp16: x = (1, 2); W_up = (3, -1), b_up = 0.5 -> u = 1.5, h = 2.25;
    W_down^T = (2, -4) -> y = (4.5, -9).  With W_up = (-3, 1): u = -0.5 -> h = 0 -> y = 0
    (the square comes after the ReLU)."""
    h16 = lambda *v: np.array(v, np.float16).view(np.uint16)
    x = h16(1, 2).reshape(1, 2)
    for w_up, y_exp, h_exp in (((3, -1), (4.5, -9.0), 2.25), ((-3, 1), (0.0, 0.0), 0.0)):
        y, h = oracle.sparse_ffn(8, 1, False, F16, np.pad(h16(*w_up), (0, 6)).reshape(1, 8),
                                 np.pad(h16(2, -4), (0, 6)).reshape(1, 8), np.pad(x, ((0, 0), (0, 6))),
                                 np.array([0], np.int32), b_up=h16(0.5), want_h=True, act=1)
        assert h[0, 0] == h_exp and np.array_equal(y[0, :2], np.array(y_exp)) and np.all(y[0, 2:] == 0)
