"""Checks of the seeded workload generator (CPU only).

The generator makes inputs, not results, so these are determinism and statistics checks:
binary16 rounding against numpy's round-to-nearest-even, independence from the thread
count, the Zipf law's defining equations, and the realized firing statistics of a generated
layer -- about 26% of neurons giving 80% of activations (PowerInfer, arXiv 2312.12456,
key results) at the configured density.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_f32_to_f16_matches_numpy_rne():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(20000) * 1e-5).astype(np.float32),          # subnormal range
        (rng.standard_normal(2000) * 7e4).astype(np.float32),            # overflow range
        np.array([0.0, -0.0, 65504.0, 65520.0, 65519.99, 2 ** -24, 2 ** -25, 2 ** -25 * 1.0000001,
                  3 * 2 ** -26, np.inf, -np.inf], dtype=np.float32),
    ])
    # exact binary16 halfway points: ties must go to even
    base = np.arange(0, 65535, 97, dtype=np.uint16).view(np.float16).astype(np.float32)
    nxt = (np.arange(0, 65535, 97, dtype=np.uint16) + 1).view(np.float16).astype(np.float32)
    mid = ((base.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)
    vals = np.concatenate([vals, mid[np.isfinite(mid)]])
    L = synth.lib()
    ours = np.array([L.ps_f32_to_f16(float(v)) for v in vals], dtype=np.uint16)
    ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_deterministic_and_thread_independent():
    a = synth.normal_f16(3, 2, synth.T_WUP, 37, 1000, 0.1)
    b = synth.normal_f16(3, 2, synth.T_WUP, 37, 1000, 0.1)
    assert np.array_equal(a, b)
    rows = np.array([36, 0, 5], dtype=np.int32)
    assert np.array_equal(synth.normal_f16(3, 2, synth.T_WUP, 3, 1000, 0.1, rows=rows), a[rows])
    q = synth.q4_0_rows(3, 2, synth.T_Q4_UP, 20, 256)
    code = ("import numpy as np, synth; "
            "a = synth.normal_f16(3, 2, synth.T_WUP, 37, 1000, 0.1); q = synth.q4_0_rows(3, 2, synth.T_Q4_UP, 20, 256); "
            "import sys; sys.stdout.buffer.write(a.tobytes() + q.tobytes())")
    env = dict(os.environ, OMP_NUM_THREADS="1", PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, check=True, cwd=ROOT).stdout
    assert out == a.tobytes() + q.tobytes()


def test_normal_moments():
    v = synth.f16_bits_to_f32(synth.normal_f16(1, 0, synth.T_P1, 256, 4096, 1.0 / 64)).astype(np.float64)
    assert abs(v.mean()) < 2e-4 and abs(v.std() * 64 - 1.0) < 5e-3
    assert np.abs(v).max() <= np.sqrt(12.0) / 64 * 1.001


def test_q4_0_rows_layout_and_variance():
    d = 1024
    rows = synth.q4_0_rows(5, 0, synth.T_Q4_DOWN, 64, d)
    assert rows.shape == (64, d * 9 // 16)
    w = np.stack([oracle.decode_row(r, oracle.Q4_0, d) for r in rows])
    codes = np.concatenate([rows[:, : d // 2] & 15, rows[:, : d // 2] >> 4])
    assert np.bincount(codes.ravel(), minlength=16).min() > 0.8 * codes.size / 16
    assert abs(w.var() * d - 1.0) < 0.05


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_zipf_solution_satisfies_its_equations(cid):
    cfg = synth.CONFIGS[cid]
    s, A = synth.zipf_solve(cfg.f, cfg.density)
    k = np.arange(1, cfg.f + 1, dtype=np.float64)
    p = np.minimum(synth.P_CAP, A * k ** -s)
    assert abs(p.mean() - cfg.density) < 1e-9
    top = int(round(synth.TOP_FRAC * cfg.f))
    assert abs(p[:top].sum() / p.sum() - synth.TOP_SHARE) < 1e-6


def test_zipf_freq_is_a_permutation_of_the_law():
    f = 4096
    s, A = synth.zipf_solve(f, 0.1)
    p, rank = synth.zipf_freq(1, 0, f, s, A)
    assert np.array_equal(np.sort(rank), np.arange(1, f + 1))
    assert np.allclose(p, np.minimum(synth.P_CAP, A * rank.astype(np.float64) ** -s))
    p2, _ = synth.zipf_freq(1, 1, f, s, A)
    assert not np.array_equal(p, p2)                 # every layer gets its own hot set


def test_hot_set_ties_by_lower_id():
    p = np.array([0.5, 0.9, 0.9, 0.1, 0.9])
    assert synth.hot_set(p, 2).tolist() == [1, 2]
    assert synth.hot_set(p, 4).tolist() == [0, 1, 2, 4]


def test_realized_firing_statistics_small_layer():
    """The 1024x4096 rank-128 layer: ~10% fire per token and the hottest 26% give ~80%."""
    cfg = synth.CONFIGS[1]
    p1, p2, c, freq = synth.make_predictor(cfg, 0)
    T = 400
    x = synth.normal_f16(cfg.seed, 0, synth.T_X, T, cfg.d, 1.0)
    _, _, tok = oracle.predict(p1, p2, c, x, want_tok_masks=True)
    fires = tok.sum(axis=0).astype(np.float64)
    density = fires.sum() / (T * cfg.f)
    assert abs(density - cfg.density) < 0.1 * cfg.density
    top = synth.hot_set(freq, int(round(0.26 * cfg.f)))
    share = fires[top].sum() / fires.sum()
    assert abs(share - 0.80) < 0.03
    assert np.corrcoef(fires / T, freq)[0, 1] > 0.95
