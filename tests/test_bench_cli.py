"""bench.py's host-side contract that needs no GPU: it measures one GPU only, so a request for more
exits with status 2 and says so (before any GPU work); the placed stack takes pi_place's resident
sets; and the kernel names it looks counter traffic up by match the committed counter records."""
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


def test_kernel_prefixes_name_the_profiled_kernels():
    """The rocprof name prefixes bench.py looks traffic up by -- the layer's kernels after the first
    predictor matrix, and the sparse FFN's -- each name a kernel in the counter record committed for
    that workload, so a renamed or re-templated kernel shows up here rather than as a silently null
    `traffic`.  The layer path and FFN form come from the C ABI's host-side queries (no GPU)."""
    import ctypes
    import glob
    import json

    sys.path.insert(0, ROOT)
    import bench
    import synth
    from activation_sparse_ffn_rank_amd import _abi

    A = 0x10000                                   # fake device addresses: the queries never dereference them
    records = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))
    assert records
    by_name = {c.name: c for c in synth.CONFIGS.values()}
    for path in records:
        with open(path) as fh:
            rec = json.load(fh)
        name, b = rec["workload"].rsplit("_b", 1)
        cfg, B = by_name[name], int(b)
        placed = cfg.hot_frac is not None
        pred = _abi.pi_predictor(cfg.d, cfg.f, cfg.r, A, A, A)
        ffn = _abi.pi_ffn(cfg.d, cfg.f, int(cfg.gated), cfg.wtype, cfg.n_hot(), A if placed else None, A, A,
                          A if cfg.bias_up else None, None, cfg.act)
        lpath = _abi.pi_layer_path(pred, ffn, B)
        _, h_kind = _abi.pi_sparse_ffn_h_offset(ffn, B)
        assert lpath in (1, 2)
        prefixes = (bench.layer_kernel_names(lpath, h_kind, B, cfg, synth, placed)[1]
                    + bench.ffn_kernel_names(h_kind, B, cfg, synth)[1])
        for pre in prefixes:
            assert any(k.startswith(pre) for k in rec["kernels"]), (rec["workload"], pre)
