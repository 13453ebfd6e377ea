#!/usr/bin/env python3
"""Decode-step benchmark of the predictor-gated sparse FFN stacks on one MI355X.

A step is one token (or one batch of B tokens) through every layer of a stack: per layer the
predictor GEMVs, the firing mask, the placement restriction and the sparse FFN over the active
neurons (pi_ffn_layer), each (layer, token) fed its own seeded input vector.  Weights and inputs
are resident in HBM before timing starts.  W warmup steps and K timed steps are replayed from HIP
graphs captured on one stream; the timed graph is replayed 5 times, each replay bracketed by HIP
events on that stream after a device synchronization, and the median is reported.

The headline (`value`) is the largest stack that fits one GPU at batch 1: 96 layers of
d_model 12288 / d_ffn 49152 with Q4_0 FFN rows (OPT-175B-shaped).  The same run measures every
other workload (the 7B-, 30B- and 40B-shaped stacks, the batch-4 and batch-8 variants, 16-token
steps of the 175B- and 7B-shaped stacks, and the single small layer) into `detail.workloads`, each
with its tokens/s, microseconds per layer and the HBM fraction of its kernels.

Printed: one JSON line.  `roofline` is the sparse-FFN kernel of the headline workload (the
kernel that reads the active rows) on its algorithmic bytes, timed with HIP events on its launch
stream around a graph of its launches; `cpu_baseline` is the CPU oracle on a bounded sample of
the same workload on this host's cores.

`python bench.py --pmc-summary WORKLOAD DIR [DIR ...]` (no GPU needed) turns rocprofv3 --pmc
output directories of runs of this script into profiles/counters_<WORKLOAD>.md and, when they hold
FETCH_SIZE and WRITE_SIZE, profiles/traffic_<WORKLOAD>.json.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
HOST_BW_GBS = 100.0            # host DRAM read bandwidth assumed by the placement policy
HEADLINE = (5, 1)              # (stack id, batch): OPT-175B-shaped Q4_0 stack at batch 1
DETAIL = ((5, 8), (5, 16), (2, 1), (2, 16), (3, 1), (3, 4), (4, 1), (1, 1))
REPS = 5                       # replays of each timed graph; the median is reported
COPY_PROBE_MIB = 256
CU_NUM = 256                   # MI355X compute units (the counter formulas divide by it)
NUM_XCC = 8                    # ... in 8 XCDs


def kernel_sources_sha256() -> str:
    """Digest of the HIP sources; hardware byte counts taken on other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "activation_sparse_ffn_rank_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel_prefixes):
    """HBM bytes per launch (read + written) summed over the kernels whose names start with one of
    kernel_prefixes, from profiles/traffic_<workload>.json -- None when there is no record, a kernel
    is missing from it, or the sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("sources_sha256") != kernel_sources_sha256():
        return None
    total = 0
    for pre in kernel_prefixes:
        hits = [v for name, v in rec.get("kernels", {}).items() if name.startswith(pre)]
        if not hits:
            return None
        total += int(hits[0]["read_bytes"]) + int(hits[0]["write_bytes"])
    return total


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=56, help="timed decode steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", type=int, default=HEADLINE[0], help="stack id (1-5) of the headline workload")
    ap.add_argument("--batch", type=int, default=HEADLINE[1])
    ap.add_argument("--layers", type=int, default=0, help="use only the first N layers (0 = all)")
    ap.add_argument("--roofline-steps", type=int, default=16, help="tokens whose launches the per-kernel legs time")
    ap.add_argument("--detail-steps", type=int, default=24, help="timed steps of each detail workload")
    ap.add_argument("--no-detail", action="store_true", help="measure the headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the measurement, run one device-to-device copy of this many MiB (a kernel of "
                         "known traffic, for scaling hardware byte counters)")
    ap.add_argument("--pmc-summary", nargs="+", metavar=("WORKLOAD", "DIR"),
                    help="summarize rocprofv3 --pmc directories into profiles/ (no GPU) and exit")
    ap.add_argument("--trace-summary", nargs=2, metavar=("WORKLOAD", "DIR"),
                    help="summarize a rocprofv3 --kernel-trace --stats directory into profiles/ (no GPU) and exit")
    ap.add_argument("--pmc-command", action="append", default=[],
                    help="with --pmc-summary: the command that made each directory (recorded in the summary)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def timed_graph(torch, stream, fn, reps=REPS):
    """Capture fn() into a graph, replay once to warm, then time `reps` replays with HIP events on
    `stream` (each after a device synchronization); returns the median elapsed ms."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del g
    return statistics.median(times), times


def ffn_kernel_names(h_kind: int, B: int, cfg, synth):
    """(label, rocprof name prefixes) of the kernels one pi_sparse_ffn call runs, by its form."""
    g = "true" if cfg.gated else "false"
    w = 1 if cfg.wtype == synth.F16 else 2
    if h_kind == 1:
        return "k_up_split + k_down_split + k_sum_split", [f"void pik::k_up_split<{B}, {g}, {w}>",
                                                         f"void pik::k_down_split<{B}, {g}, {w}, false>",
                                                         "pik::k_sum_split("]
    if h_kind == 2:
        return "k_sparse_up + k_sparse_down", [f"void pik::k_sparse_up<{B}, {g}, {w}>", f"void pik::k_sparse_down<{B}, {w}>"]
    if h_kind == 3:
        if cfg.wtype != synth.F16:                              # x re-laid out for the Q4_0 MFMA operands first
            return "k_wide_xmf + k_wide_up_q4 + k_wide_down", ["pik::k_wide_xmf(", "pik::k_wide_up_q4(",
                                                               "void pik::k_wide_down<"]
        if B > 8:                                               # fp16 rows: x re-laid out past 8 tokens
            return "k_wide_xmf + k_wide_up + k_wide_down", ["pik::k_wide_xmf(", "void pik::k_wide_up<",
                                                            "void pik::k_wide_down<"]
        return "k_wide_up + k_wide_down", ["void pik::k_wide_up<", "void pik::k_wide_down<"]
    return f"kind {h_kind}", []


def layer_kernel_names(path: int, h_kind: int, B: int, cfg, synth, placed: bool):
    """(label, rocprof name prefixes) of the kernels one pi_ffn_layer_from_hidden call runs (the layer
    after the first predictor matrix), by the layer's path and its sparse FFN form."""
    ffn_label, ffn_prefixes = ffn_kernel_names(h_kind, B, cfg, synth)
    g = "true" if cfg.gated else "false"
    w = 1 if cfg.wtype == synth.F16 else 2
    if path == 1:
        rest_label, rest_prefixes = "k_layer_tail", [f"void pik::k_layer_tail<{B}, {g}, {w},"]
    elif h_kind == 1:
        # the layer's own form at batch <= 2: logits, mask and up rows in one kernel, then the down
        # rows on h by neuron id
        rest_label = "k_pred_up + k_down_split + k_sum_split"
        rest_prefixes = [f"void pik::k_pred_up<{B}, {g}, {w},", f"void pik::k_down_split<{B}, {g}, {w}, true>",
                         "pik::k_sum_split("]
    else:
        # the second predictor matrix on MFMA from batch 3 (d_ffn >= 16384) or 6 (z staged in LDS up
        # to rank 1024), then the list from its flag words; the staged kernel's grid also lays out x
        # for the Q4_0 up step, so the layer runs no k_wide_xmf of its own
        mfma = B >= (3 if cfg.f >= 16384 else 6)
        pl2 = ("k_pred_l2_mfma_s" if cfg.r <= 1024 else "k_pred_l2_mfma") if mfma else "k_pred_l2"
        in_label, in_prefixes = ffn_label, ffn_prefixes
        q4_wide = h_kind == 3 and cfg.wtype != synth.F16
        if mfma and cfg.r <= 1024 and h_kind == 3:
            # the staged predictor's grid lays out x: no k_wide_xmf launch in the layer
            in_label = in_label.replace("k_wide_xmf + ", "")
            in_prefixes = [q for q in in_prefixes if q != "pik::k_wide_xmf("]
        # with every neuron resident, the Q4_0 up step lists the positions from the flag words itself
        cb_label, cb_prefixes = ("", []) if (q4_wide and not placed) else ("k_compact_bits + ", ["pik::k_compact_bits("])
        rest_label = f"{pl2} + {cb_label}{in_label}"
        rest_prefixes = [f"void pik::{pl2}<"] + cb_prefixes + in_prefixes
    return rest_label, rest_prefixes


# ---------------------------------------------------------------------------------- one workload

def measure(torch, synth, _abi, cfg, layers, B, W, K, R, dev, stream, *, wide=False, hots=None):
    """Time K decode steps of `layers` at batch B (median of REPS graph replays) and the per-kernel
    legs; returns the workload's record (plus private fields starting with '_')."""
    L = len(layers)
    tokens = W + K
    x_all = synth.make_x_all(cfg, L, tokens, B)                 # [T][L][B][d] fp16 bits
    xd = torch.from_numpy(x_all.view(np.int16)).to(dev)
    # one workspace per group of layers whose FFN descriptors agree (placed layers may hold different
    # counts of neurons, and a workspace may serve several layers only when their shapes agree)
    wss = {}

    def ws_of(lay):
        if lay.n_slots not in wss:
            wss[lay.n_slots] = lay.workspace(B, device=dev)
        return wss[lay.n_slots]

    for lay in layers:
        ws_of(lay)
    y = torch.empty((L, B, cfg.d), dtype=torch.float32, device=dev)

    def step(t):
        for l in range(L):
            lay = layers[l]
            _abi.pi_ffn_layer(lay.pred, lay.ffn, xd[t, l], B, y[l], None, None, None, ws_of(lay))

    with torch.cuda.stream(stream):
        step(0)
        torch.cuda.synchronize()

        def warm():
            for t in range(W):
                step(t)

        def timed():
            for t in range(W, W + K):
                step(t)

        g_warm = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_warm, stream=stream):
            warm()
        g_warm.replay()
        torch.cuda.synchronize()
        del g_warm
        elapsed_ms, rep_ms = timed_graph(torch, stream, timed)
    for w in wss.values():
        if _abi.workspace_status(w) != 0:
            raise RuntimeError(f"workspace status {_abi.workspace_status(w)}: a cross-workgroup wait timed out")

    # ---- per-kernel legs.  pi_ffn_layer = pi_predict_hidden (z = ReLU(P1 x)) followed by
    # pi_ffn_layer_from_hidden (logits, mask and the sparse FFN).  An eager pass runs both on R tokens
    # x L layers, keeping every z and index list, and runs pi_sparse_ffn on each list (the sparse FFN
    # alone) to count the listed neurons whose h is nonzero for some token.  Each entry point's R*L
    # launches are then captured into a graph of their own and timed (median of REPS replays).
    R = min(R, K)
    N = R * L
    rb = cfg.row_bytes()
    in_rows = 2 if cfg.gated else 1
    pred_bytes = 2 * (cfg.r * cfg.d + cfg.f * cfg.r + cfg.f)
    path = _abi.pi_layer_path(layers[0].pred, layers[0].ffn, B)
    z_all = torch.empty((N, B, cfg.r), dtype=torch.float32, device=dev)
    masks = torch.empty((N, cfg.f), dtype=torch.uint8, device=dev)
    idx_all = torch.empty((N, cfg.f), dtype=torch.int32, device=dev)
    cnt_all = torch.empty((N, 2), dtype=torch.int32, device=dev)
    # placed layers may hold different counts of neurons: size for the largest
    ws_f = torch.zeros(max(_abi.pi_workspace_bytes(None, lay.ffn, B) for lay in layers), dtype=torch.uint8,
                       device=dev)
    y_chk = torch.empty((B, cfg.d), dtype=torch.float32, device=dev)
    ar = torch.arange(max(lay.n_slots for lay in layers), device=dev)
    cases = [(W + i // L, i % L) for i in range(N)]             # (token, layer) of launch i

    def run_hidden():
        for i, (t, l) in enumerate(cases):
            _abi.pi_predict_hidden(layers[l].pred, xd[t, l], B, z_all[i])

    def run_rest():
        for i, (t, l) in enumerate(cases):
            _abi.pi_ffn_layer_from_hidden(layers[l].pred, layers[l].ffn, xd[t, l], B, z_all[i], y_chk, None, None,
                                          None, ws_of(layers[l]))

    def run_sparse():
        for i, (t, l) in enumerate(cases):
            _abi.pi_sparse_ffn(layers[l].ffn, xd[t, l], B, idx_all[i], cnt_all[i], y_chk, ws_f)

    with torch.cuda.stream(stream):
        run_hidden()
        for i, (t, l) in enumerate(cases):
            _abi.pi_ffn_layer_from_hidden(layers[l].pred, layers[l].ffn, xd[t, l], B, z_all[i], y_chk, masks[i],
                                          idx_all[i], cnt_all[i], ws_of(layers[l]))
        live = []
        for i, (t, l) in enumerate(cases):
            _abi.pi_sparse_ffn(layers[l].ffn, xd[t, l], B, idx_all[i], cnt_all[i], y_chk, ws_f)
            ns = layers[l].n_slots
            h, ok = _abi.sparse_ffn_h(layers[l].ffn, B, ws_f, ns)
            live.append(((h != 0).any(dim=0) & ok & (ar[:ns] < cnt_all[i, 0])).sum())
        torch.cuda.synchronize()
        n_live = torch.stack(live).cpu().numpy().astype(np.float64)
        cnt_host = cnt_all.cpu().numpy().astype(np.float64)
        leg_us = {}
        for name, fn in (("hidden", run_hidden), ("rest", run_rest), ("sparse_ffn", run_sparse)):
            ms, _ = timed_graph(torch, stream, fn)
            leg_us[name] = ms * 1000.0 / N
    for w in list(wss.values()) + [ws_f]:
        if _abi.workspace_status(w) != 0:
            raise RuntimeError("workspace status nonzero: a cross-workgroup wait timed out")
    n_act, n_pred = cnt_host[:, 0], cnt_host[:, 1]
    vec_bytes = B * cfg.d * (2 + 4) + 2 * cfg.d                  # x in, y out, b_down
    slot_bytes = 4 * cfg.f if layers[0].slot_of is not None else 0
    _, h_kind = _abi.pi_sparse_ffn_h_offset(layers[0].ffn, B)
    # rows the sparse FFN reads: every listed input row; the down rows of every listed neuron except
    # in the GEMV two-kernel form, which skips those whose h is zero for every token
    n_read_down = n_live if h_kind == 2 else n_act
    ffn_touched = n_act * in_rows * rb + n_read_down * rb + 8 * n_act + vec_bytes
    ffn_predicted = n_act * (in_rows + 1) * rb + 8 * n_act + vec_bytes
    # the rest of the layer: P2 and c, z, every listed input row, and the down rows the form reads --
    # at batch <= 2 (k_pred_up) only those whose h is nonzero for some token
    pred_up = path == 2 and h_kind == 1
    rest_down = n_live if (pred_up or h_kind == 2) else n_act
    rest_bytes = (2 * cfg.f * cfg.r + 2 * cfg.f + 4 * B * cfg.r + slot_bytes + n_act * in_rows * rb + rest_down * rb
                  + vec_bytes)
    hidden_bytes = 2 * cfg.r * cfg.d + 2 * B * cfg.d + 4 * B * cfg.r
    ffn_label, ffn_prefixes = ffn_kernel_names(h_kind, B, cfg, synth)
    rest_label, rest_prefixes = layer_kernel_names(path, h_kind, B, cfg, synth, placed=hots is not None)
    step_bytes = (pred_bytes + float(ffn_touched.mean())) * L
    ms_per_step = elapsed_ms / K

    def gbs(nbytes, us):
        return nbytes / (us * 1e-6) / 1e9

    rec = {
        "workload": f"{cfg.name}_b{B}",
        "description": describe(cfg, L, B, synth),
        "batch": B, "layers": L, "steps": K, "warmup": W,
        "tokens_per_s": round(B * K / (elapsed_ms / 1e3), 2),
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_replays": [round(t / K, 4) for t in rep_ms],
        "us_per_layer": round(ms_per_step * 1000.0 / L, 3),
        "step_gb_algorithmic": round(step_bytes / 1e9, 4),
        "step_gbs": round(step_bytes / 1e9 / (ms_per_step / 1e3), 1),
        "step_hbm_frac": round(step_bytes / 1e9 / (ms_per_step / 1e3) / PEAK_HBM_GBS, 4),
        "layer_path": path,
        "kernels": {
            "predict_hidden": {"kernel": "k_pred_l1", "us": round(leg_us["hidden"], 3), "bytes": hidden_bytes,
                               "gbs": round(gbs(hidden_bytes, leg_us["hidden"]), 1),
                               "frac": round(gbs(hidden_bytes, leg_us["hidden"]) / PEAK_HBM_GBS, 4)},
            "layer_from_hidden": {"kernel": rest_label, "us": round(leg_us["rest"], 3),
                                  "bytes": round(float(rest_bytes.mean())),
                                  "gbs": round(gbs(float(rest_bytes.mean()), leg_us["rest"]), 1),
                                  "frac": round(gbs(float(rest_bytes.mean()), leg_us["rest"]) / PEAK_HBM_GBS, 4)},
            "sparse_ffn": {"kernel": ffn_label, "us": round(leg_us["sparse_ffn"], 3),
                           "bytes": round(float(ffn_touched.mean())),
                           "bytes_predicted_rows": round(float(ffn_predicted.mean())),
                           "gbs": round(gbs(float(ffn_touched.mean()), leg_us["sparse_ffn"]), 1),
                           "frac": round(gbs(float(ffn_touched.mean()), leg_us["sparse_ffn"]) / PEAK_HBM_GBS, 4)},
        },
        "predictor_bytes": pred_bytes,
        "active_density": round(float(n_act.mean()) / cfg.f, 4),
        "predicted_density": round(float(n_pred.mean()) / cfg.f, 4),
        "covered_share": round(float(n_act.sum() / max(n_pred.sum(), 1)), 4),
        "down_rows_zero_h_share": round(1.0 - float(n_live.sum()) / max(float(n_act.sum()), 1.0), 4),
        "_ffn_prefixes": ffn_prefixes, "_rest_prefixes": rest_prefixes,
        "_ffn": (float(ffn_touched.mean()), leg_us["sparse_ffn"], ffn_label, N),
        "_rest": (float(rest_bytes.mean()), leg_us["rest"], rest_label, N),
    }
    if hots is not None:
        rec["cold_host"] = cold_leg(torch, synth, _abi, cfg, layers, hots, B, x_all, xd, masks, cases, ws_of, stream,
                                    dev, ms_per_step)
    if wide and B == 1 and R >= 16 and layers[0].slot_of is None:
        rec["wide_b16"] = wide_leg(torch, _abi, cfg, layers, xd, masks, cases, stream, dev, in_rows, rb)
    del xd, z_all, masks, idx_all, ws_f, wss
    return rec


def describe(cfg, L, B, synth):
    return (f"{cfg.name}: {L} layers, d_model={cfg.d}, d_ffn={cfg.f}, predictor rank {cfg.r}, "
            f"{'ReGLU' if cfg.gated else 'ReLU'}, {'fp16' if cfg.wtype == synth.F16 else 'Q4_0'} weights, "
            f"batch {B}, Zipf firing at {cfg.density:.0%} target density"
            + (f", resident set placed by pi_place under a {cfg.hot_frac:.0%} budget" if cfg.hot_frac else ""))


def place_stack(synth, _abi, cfg, L):
    """Resident neurons of every layer, chosen by pi_place (offline policy over the firing
    frequencies, the per-neuron bytes and the two memories' bandwidths) under a device budget of
    cfg.hot_frac of the stack's FFN bytes.  Returns (ascending resident ids per layer, summary), or
    (None, None) for a stack that is wholly resident."""
    if cfg.hot_frac is None:
        return None, None
    nb = (3 if cfg.gated else 2) * cfg.row_bytes()
    freqs = [synth.layer_freq(cfg, l) for l in range(L)]
    budget = int(round(cfg.hot_frac * L * cfg.f * nb))
    slot_ofs, n_placed, t_exp = _abi.pi_place([cfg.f] * L, [nb] * L, freqs, budget, PEAK_HBM_GBS * 1e9,
                                              HOST_BW_GBS * 1e9)
    hots = [np.flatnonzero(so >= 0).astype(np.int32) for so in slot_ofs]
    share = n_placed / cfg.f
    expected_rows = sum(float(fr[h].sum()) for fr, h in zip(freqs, hots))
    all_rows = sum(float(fr.sum()) for fr in freqs)
    return hots, {"policy": "pi_place", "budget_share": cfg.hot_frac, "budget_gb": round(budget / 1e9, 3),
                  "resident_share": round(float(n_placed.sum()) / (L * cfg.f), 4),
                  "resident_share_min": round(float(share.min()), 4), "resident_share_max": round(float(share.max()), 4),
                  "expected_covered_share": round(expected_rows / all_rows, 4),
                  "bandwidths_gbs": {"gpu": PEAK_HBM_GBS, "host": HOST_BW_GBS},
                  "expected_us_per_token": round(t_exp * 1e6, 2)}


def cold_leg(torch, synth, _abi, cfg, layers, hots, B, x_all, xd, masks, cases, ws_of, stream, dev, ms_per_step):
    """Host half of the hybrid split: the predicted neurons that are not resident, computed by
    pi_cold_ffn_host on the masks the device produced (first two layers), and the hybrid layer end
    to end (device layer -> mask to pinned host memory -> host half -> host y added on the device)."""
    L = len(layers)
    in_rows = 2 if cfg.gated else 1
    n_lay = min(L, 2)
    masks_h = masks.cpu().numpy()
    hosts = []
    for l in range(n_lay):
        cold_ids = np.setdiff1d(np.arange(cfg.f, dtype=np.int32), hots[l])
        w_in_c, w_dn_c, b_up_c, _ = synth.make_ffn(cfg, l, cold_ids)
        slot_c = np.full(cfg.f, -1, np.int32)
        slot_c[cold_ids] = np.arange(cold_ids.size, dtype=np.int32)
        hosts.append(_abi.HostFFN(w_in_c, w_dn_c, d_model=cfg.d, d_ffn=cfg.f, gated=cfg.gated, wtype=cfg.wtype,
                                  slot_of=slot_c, b_up=b_up_c))
    ws_h = np.zeros(_abi.pi_cold_workspace_bytes(hosts[0], B), np.uint8)
    y_h = np.empty((B, cfg.d), np.float32)
    # every host thread, and half of them (hosts that expose two threads per core often run this
    # memory-bound loop faster on one per core); the faster is reported, with its count
    best = None
    for nthr in sorted({synth.num_threads(), max(1, synth.num_threads() // 2)}):
        times, counts_c = [], []
        for i, (t, l) in enumerate(cases):
            if l >= n_lay:
                continue
            x_h = np.ascontiguousarray(x_all[t, l])
            s0 = time.perf_counter()
            counts_c.append(_abi.pi_cold_ffn_host(hosts[l], x_h, B, masks_h[i], y_h, ws_h, nthr))
            times.append(time.perf_counter() - s0)
        med = float(np.median(times))
        if best is None or med < best[0]:
            best = (med, nthr, counts_c, len(times))
    nthr = best[1]
    mask_pin = torch.empty(cfg.f, dtype=torch.uint8, pin_memory=True)
    ycold_pin = torch.empty((B, cfg.d), dtype=torch.float32, pin_memory=True)
    y_dev = torch.empty((B, cfg.d), dtype=torch.float32, device=dev)
    m_dev = torch.empty(cfg.f, dtype=torch.uint8, device=dev)
    yc_dev = torch.empty((B, cfg.d), dtype=torch.float32, device=dev)
    hyb = []
    with torch.cuda.stream(stream):
        for rep in range(2):
            for i, (t, l) in enumerate(cases):
                if l >= n_lay:
                    continue
                torch.cuda.synchronize()
                s0 = time.perf_counter()
                _abi.pi_ffn_layer(layers[l].pred, layers[l].ffn, xd[t, l], B, y_dev, m_dev, None, None,
                                  ws_of(layers[l]))
                mask_pin.copy_(m_dev, non_blocking=True)
                stream.synchronize()
                _abi.pi_cold_ffn_host(hosts[l], np.ascontiguousarray(x_all[t, l]), B, mask_pin.numpy(),
                                      ycold_pin.numpy(), ws_h, nthr)
                yc_dev.copy_(ycold_pin, non_blocking=True)
                y_dev.add_(yc_dev)
                stream.synchronize()
                if rep == 1:
                    hyb.append(time.perf_counter() - s0)
    rb = cfg.row_bytes()
    return {"host_us_per_layer": round(1e6 * best[0], 2), "neurons_per_layer": round(float(np.mean(best[2])), 1),
            "rows_mb_per_layer": round(float(np.mean(best[2])) * (in_rows + 1) * rb / 1e6, 3),
            "threads": best[1], "calls": best[3],
            "hybrid_layer_us": round(1e6 * float(np.median(hyb)), 2),
            "device_only_layer_us": round(ms_per_step * 1000.0 / L, 2)}


def wide_leg(torch, _abi, cfg, layers, xd, masks, cases, stream, dev, in_rows, rb):
    """pi_sparse_ffn_wide over each layer's union of 16 tokens' predicted lists (the masks of the
    eager pass, ORed and compacted outside the timed region), x of those 16 tokens."""
    L = len(layers)
    with torch.cuda.stream(stream):
        idx_w = torch.empty((L, cfg.f), dtype=torch.int32, device=dev)
        cnt_w = torch.empty((L, 2), dtype=torch.int32, device=dev)
        x_w = torch.empty((L, 16, cfg.d), dtype=torch.int16, device=dev)
        for l in range(L):
            sel = [i for i, (t, ll) in enumerate(cases) if ll == l][:16]
            union = masks[sel].amax(dim=0).contiguous()
            _abi.pi_compact(union, cfg.f, None, idx_w[l], cnt_w[l])
            x_w[l] = xd[[cases[i][0] for i in sel], l, 0]
        ws_w = torch.empty(_abi.pi_sparse_ffn_wide_workspace_bytes(layers[0].ffn, 16), dtype=torch.uint8, device=dev)
        y_w = torch.empty((16, cfg.d), dtype=torch.float32, device=dev)

        def run_wide():
            for l in range(L):
                _abi.pi_sparse_ffn_wide(layers[l].ffn, x_w[l], 16, idx_w[l], cnt_w[l], y_w, ws_w)

        ms, _ = timed_graph(torch, stream, run_wide)
        wide_us = ms * 1000.0 / L
    n_w = cnt_w[:, 0].cpu().numpy().astype(np.float64)
    q4 = rb < 2 * cfg.d                                          # Q4_0 rows are shorter than fp16 ones
    wide_bytes = float((n_w * (in_rows + 1) * rb + 4 * n_w).mean()) + 16 * cfg.d * (2 + 4) + 2 * cfg.d
    return {"batch": 16, "us_per_layer": round(wide_us, 3), "neurons_per_layer": round(float(n_w.mean()), 1),
            "algorithmic_bytes_per_layer": int(wide_bytes),
            "gbs": round(wide_bytes / (wide_us * 1e-6) / 1e9, 1),
            "hbm_frac": round(wide_bytes / (wide_us * 1e-6) / 8e12, 4),
            "kernels": ("k_wide_xmf + k_wide_up_q4" if q4 else "k_wide_up") + " + k_wide_down (pi_sparse_ffn_wide, MFMA f16)"}


def cpu_oracle(synth, oracle, cfg, L, B, tokens, budget_s, threads=None):
    """The oracle's whole layer (predictor, mask, compaction, sparse FFN) on layers 0..3 of the stack,
    cycling over the seeded tokens until `budget_s` seconds of wall time, scaled to an L-layer step."""
    if threads is not None:
        oracle.set_num_threads(threads)
    n_lay = min(L, 4)
    hosts = [synth.make_layer(cfg, l) for l in range(n_lay)]
    x_all = synth.make_x_all(cfg, n_lay, tokens, B)
    done, spent, t = 0, 0.0, 0
    while spent < budget_s:
        for l in range(n_lay):
            s0 = time.perf_counter()
            oracle.ffn_layer(hosts[l], x_all[t % tokens, l], want_logits=False)
            spent += time.perf_counter() - s0
            done += 1
        t += 1
    used = oracle.num_threads()
    per_layer = spent / done
    return {"value": round(B / (per_layer * L), 3), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} evaluations of the whole layer (predictor, mask, compaction, sparse FFN over the "
                      f"listed neurons, fp64) at batch {B} on {used} threads of {cpu_model()}: layers 0..{n_lay - 1} "
                      f"of the {cfg.name} stack, {t} token steps cycling over {tokens} seeded inputs; {spent:.1f}s, "
                      f"{per_layer * 1e3:.2f} ms per layer, scaled to the {L}-layer step"}


# ---------------------------------------------------------------------------------- counters

def pmc_summary(args):
    """Summarize rocprofv3 --pmc output directories (runs of this script) per kernel."""
    import collections
    import csv
    import glob
    workload, dirs = args.pmc_summary[0], args.pmc_summary[1:]
    vals = collections.defaultdict(lambda: collections.defaultdict(list))   # counter -> kernel -> values
    probe = {}
    for dd in dirs:
        files = glob.glob(os.path.join(dd, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {dd}")
        rows = [r for f in files for r in csv.DictReader(open(f))]
        for r in rows:
            vals[r["Counter_Name"]][r["Kernel_Name"]].append(float(r["Counter_Value"]))
        # the copy probe is the last device copy of the run (COPY_PROBE_MIB MiB read and written)
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"] or "copy" in r["Kernel_Name"].lower()]
        for cname in ("FETCH_SIZE", "WRITE_SIZE"):
            cr = [r for r in copies if r["Counter_Name"] == cname]
            if cr:
                last = max(cr, key=lambda r: int(r["Dispatch_Id"]))
                probe[cname] = (last["Kernel_Name"], float(last["Counter_Value"]))
    ours = sorted({k for c in vals.values() for k in c if k.startswith(("void pik::", "pik::"))})
    probe_kib = COPY_PROBE_MIB * 1024
    scale = {c: probe_kib / v for c, (_, v) in probe.items() if v > 0}
    lines = [f"# Hardware counters per dispatch: {workload}", "",
             "Commands (from the repository root; one counter group per run):", "", "```"]
    lines += args.pmc_command or ["(not recorded)"]
    lines += ["```", "", f"Sources sha256: `{kernel_sources_sha256()}`", ""]
    if scale:
        lines.append("Calibration: the last device copy of each run moves "
                     f"{COPY_PROBE_MIB} MiB ({probe_kib} KiB) read and written; "
                     + ", ".join(f"{c} reads {probe[c][1]:.0f} KiB for it (scale {scale[c]:.3f})" for c in scale) + ".")
        lines.append("")
    counters = sorted(vals)
    lines.append("| kernel | dispatches | " + " | ".join(counters) + " |")
    lines.append("|---|---:|" + "---:|" * len(counters))
    for k in ours:
        n = max(len(vals[c].get(k, [])) for c in counters)
        cells = []
        for c in counters:
            v = vals[c].get(k)
            cells.append(f"{sum(v) / len(v):.4g}" if v else "")
        lines.append(f"| `{k[:90]}` | {n} | " + " | ".join(cells) + " |")
    derived = []
    for k in ours:
        d = {}
        mean = lambda c: (sum(vals[c][k]) / len(vals[c][k])) if k in vals.get(c, {}) else None
        if mean("FETCH_SIZE") is not None and "FETCH_SIZE" in scale:
            d["read MB"] = mean("FETCH_SIZE") * 1024 * scale["FETCH_SIZE"] / 1e6
        if mean("WRITE_SIZE") is not None and "WRITE_SIZE" in scale:
            d["written MB"] = mean("WRITE_SIZE") * 1024 * scale["WRITE_SIZE"] / 1e6
        hit, miss = mean("TCC_HIT_sum"), mean("TCC_MISS_sum")
        if hit is not None and miss is not None and hit + miss > 0:
            d["L2 hit rate"] = hit / (hit + miss)
        wc, gui = mean("SQ_WAVE_CYCLES"), mean("GRBM_GUI_ACTIVE")
        if gui:
            gui /= NUM_XCC                    # the CSV sums the per-XCD busy counters; the formula takes one
        if wc is not None and gui:
            # rocprofv3's OccupancyPercent: 400 * SQ_WAVE_CYCLES / GRBM_GUI_ACTIVE / CU_NUM / 32
            d["occupancy %"] = 400.0 * wc / gui / CU_NUM / 32.0
            d["mean resident waves per CU"] = 4.0 * wc / gui / CU_NUM
        iv = mean("SQ_INSTS_VALU")
        if iv is not None and mean("SQ_WAVES"):
            d["VALU instructions per wave"] = iv / mean("SQ_WAVES")
        if gui:
            d["GPU busy cycles per XCD"] = gui
        if d:
            derived.append((k, d))
    if derived:
        lines += ["", "Derived (means over the dispatches above):", ""]
        for k, d in derived:
            lines.append(f"- `{k[:90]}`: " + ", ".join(f"{n} {v:.4g}" for n, v in d.items()))
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"counters_{workload}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    if "FETCH_SIZE" in scale and "WRITE_SIZE" in scale:
        kernels = {}
        for k in ours:
            f = vals["FETCH_SIZE"].get(k)
            w = vals["WRITE_SIZE"].get(k)
            if f and w:
                kernels[k] = {"read_bytes": int(round(sum(f) / len(f) * 1024 * scale["FETCH_SIZE"])),
                              "write_bytes": int(round(sum(w) / len(w) * 1024 * scale["WRITE_SIZE"]))}
        rec = {"workload": workload, "sources_sha256": kernel_sources_sha256(), "fetch_scale": scale["FETCH_SIZE"],
               "write_scale": scale["WRITE_SIZE"], "commands": args.pmc_command, "kernels": kernels}
        with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
    print("\n".join(lines))


def trace_summary(args):
    """Summarize a rocprofv3 --kernel-trace --stats directory (a run of this script) per kernel."""
    import csv
    import glob
    workload, dd = args.trace_summary
    files = glob.glob(os.path.join(dd, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {dd}")
    rows = list(csv.DictReader(open(files[0])))
    lines = [f"# Kernel trace: {workload}", "", "Command (from the repository root):", "", "```"]
    lines += args.pmc_command or ["(not recorded)"]
    lines += ["```", "", f"Sources sha256: `{kernel_sources_sha256()}`", "",
              "| kernel | calls | average us | min us | max us | share of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.2f}% |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{workload}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ---------------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.trace_summary:
        trace_summary(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the sparse-FFN hot path has no multi-GPU leg "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from activation_sparse_ffn_rank_amd import DeviceLayer, _abi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    head = (args.config, args.batch)
    plan = [head] + ([] if args.no_detail else [w for w in DETAIL if w != head])
    # one stack at a time: every batch of a stack is measured on the same resident layers
    order = []
    for cid, _ in plan:
        if cid not in order:
            order.append(cid)
    results = {}
    for cid in order:
        cfg = synth.CONFIGS[cid]
        L = cfg.layers if args.layers <= 0 else min(args.layers, cfg.layers)
        t0 = time.time()
        hots, placement = place_stack(synth, _abi, cfg, L)
        layers = []
        for l in range(L):
            host = synth.make_layer(cfg, l, hot=None if hots is None else hots[l])
            layers.append(DeviceLayer.from_host(host, device=dev))
            del host
        torch.cuda.synchronize()
        log(f"stack {cfg.cid} ({cfg.name}): {L} layers generated and resident in {time.time() - t0:.1f}s")
        for wcid, B in plan:
            if wcid != cid:
                continue
            is_head = (wcid, B) == head
            if is_head:
                W, K = args.warmup, args.steps
            else:
                W, K = 4, max(1, min(args.detail_steps, cfg.tokens - 4))
            rec = measure(torch, synth, _abi, cfg, layers, B, W, K, args.roofline_steps, dev, stream,
                          wide=(cid in (2, 5)), hots=hots)
            if placement is not None:
                rec["placement"] = placement
            results[(wcid, B)] = rec
            log(f"{rec['workload']}: {rec['tokens_per_s']} tokens/s, {rec['us_per_layer']} us/layer, sparse FFN "
                f"{rec['kernels']['sparse_ffn']['us']} us ({rec['kernels']['sparse_ffn']['frac']} of HBM peak)")
        del layers
        torch.cuda.empty_cache()

    h = results[head]
    cfg = synth.CONFIGS[head[0]]
    L = h["layers"]
    # the roofline: the launches of pi_ffn_layer_from_hidden (second predictor matrix, mask, sparse FFN:
    # the step's dominant kernels, most of its time); beside it the sparse FFN alone on the same lists
    # (the metric's GB/s on active-row bytes)
    rest_b, rest_us, rest_label, rest_n = h["_rest"]
    roof_traffic = measured_traffic(h["workload"], h["_rest_prefixes"]) if L == cfg.layers else None
    roof_gbs = rest_b / (rest_us * 1e-6) / 1e9
    ffn_bytes, ffn_us, ffn_label, ffn_n = h["_ffn"]
    ffn_traffic = measured_traffic(h["workload"], h["_ffn_prefixes"]) if L == cfg.layers else None
    ffn_gbs = ffn_bytes / (ffn_us * 1e-6) / 1e9

    cpu = None
    c1_single = None
    if not args.no_cpu_baseline:
        import oracle
        cpu = cpu_oracle(synth, oracle, cfg, L, head[1], cfg.tokens, args.cpu_seconds)
        if not args.no_detail:
            # the single small layer on one thread (all of its seeded tokens), as a fixed reference
            c1 = synth.CONFIGS[1]
            n_all = oracle.num_threads()
            oracle.set_num_threads(1)
            lay = synth.make_layer(c1, 0)
            xs = synth.make_x_all(c1, 1, c1.tokens, 1)
            s0 = time.perf_counter()
            for t in range(c1.tokens):
                oracle.ffn_layer(lay, xs[t, 0], want_logits=False)
            c1_s = time.perf_counter() - s0
            oracle.set_num_threads(n_all)
            c1_single = {"stack": c1.name, "tokens": c1.tokens, "threads": 1, "seconds": round(c1_s, 3),
                         "tokens_per_s": round(c1.tokens / c1_s, 2), "cpu_model": cpu_model()}

    def public(rec):
        return {k: v for k, v in rec.items() if not k.startswith("_")}

    out = {
        "metric": "sparse-FFN decode tokens/s (batch 1) + achieved HBM GB/s on active-row bytes",
        "value": h["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": h["steps"],
        "warmup": h["warmup"],
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_0" if cfg.wtype == synth.Q4_0 else "f16",
        "data": "synthetic",
        "config": {
            "workload": h["description"],
            "global_batch": head[1], "layers": L, "d_model": cfg.d, "d_ffn": cfg.f, "rank": cfg.r,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": f"{rest_label} (pi_ffn_layer_from_hidden: second predictor matrix, mask, the listed "
                      f"neurons' up rows, the down rows they need)",
            "achieved": round(roof_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(roof_gbs / PEAK_HBM_GBS, 4),
            "traffic": roof_traffic,
            "bytes_per_launch": round(rest_b),
            "launch_us": round(rest_us, 3),
            "launches": int(rest_n),
        },
        "active_rows": {
            "kernel": f"{ffn_label} (pi_sparse_ffn on the same lists: the listed neurons' up rows with bias "
                      f"and ReLU, their rows of W_down^T)",
            "achieved": round(ffn_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(ffn_gbs / PEAK_HBM_GBS, 4),
            "traffic": ffn_traffic,
            "bytes_per_launch": round(ffn_bytes),
            "launch_us": round(ffn_us, 3),
            "launches": int(ffn_n),
        },
        "cpu_baseline": cpu,
        "detail": {
            "headline": public(h),
            "workloads": [public(results[w]) for w in plan if w != head],
            "cpu_c1_single_thread": c1_single,
            "timing": f"median of {REPS} replays of each timed graph (HIP events on the launch stream)",
        },
    }
    print(json.dumps(out), flush=True)
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe_mib} MiB read and written")


if __name__ == "__main__":
    main()
