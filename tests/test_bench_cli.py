"""bench.py's command-line contract that needs no GPU: it measures one GPU only, so a request for
more exits with status 2 and says so (before any GPU work)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_placed_stack_takes_pi_place_resident_sets():
    """The hot-resident stack's layers get their resident neurons from pi_place under the stack's
    budget (host only): ascending ids, within the budget, and the hottest neurons kept."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    import synth
    from activation_sparse_ffn_rank_amd import _abi
    cfg = synth.CONFIGS[4]
    L = 3
    hots, summary = bench.place_stack(synth, _abi, cfg, L)
    nb = 2 * cfg.row_bytes()
    assert len(hots) == L and summary["policy"] == "pi_place"
    assert sum(h.size for h in hots) * nb <= cfg.hot_frac * L * cfg.f * nb + 1
    for l, h in enumerate(hots):
        assert np.all(np.diff(h) > 0)
        p = synth.layer_freq(cfg, l)
        cold = np.setdiff1d(np.arange(cfg.f), h)
        assert p[h].min() >= p[cold].max()                 # the most frequent neurons are the resident ones
    assert bench.place_stack(synth, _abi, synth.CONFIGS[2], 2) == (None, None)
