#!/usr/bin/env python3
"""Decode-step benchmark of the predictor-gated sparse FFN stack on one MI355X.

A step is one token (or one batch of B tokens) through every layer of the stack: per layer the
predictor GEMVs, the firing mask and its compaction, and the sparse FFN over the active neurons
(pi_ffn_layer), with each (layer, token) fed its own seeded input vector.  Inputs and weights
are resident in HBM before timing starts.  W warmup steps and K timed steps are replayed from
HIP graphs captured on one stream; the timed region is bracketed by device synchronizations.

Printed: one JSON line with tokens/s, ms per step, per-layer microseconds, the roofline of the
sparse-FFN kernels on the bytes they must read (HIP events on the launch stream, eager pass),
and the CPU oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128, help="timed decode steps (tokens per sequence)")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", type=int, default=2, help="layer-stack configuration id (1-5)")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--layers", type=int, default=0, help="use only the first N layers (0 = all)")
    ap.add_argument("--roofline-steps", type=int, default=32, help="eager steps timed per kernel group")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph replay")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the sparse-FFN hot path has no multi-GPU leg "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from activation_sparse_ffn_rank_amd import DeviceLayer, _abi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = synth.CONFIGS[args.config]
    B = args.batch
    L = cfg.layers if args.layers <= 0 else min(args.layers, cfg.layers)
    K, W = args.steps, args.warmup
    dev = torch.device("cuda:0")

    # ------------------------------------------------------------------ weights and inputs
    t0 = time.time()
    layers = []
    for l in range(L):
        host = synth.make_layer(cfg, l)
        layers.append(DeviceLayer.from_host(host, device=dev))
        del host
    x_all = synth.make_x_all(cfg, L, W + K, B)                  # [T][L][B][d] fp16 bits
    xd = torch.from_numpy(x_all.view(np.int16)).to(dev)
    torch.cuda.synchronize()
    log(f"config {cfg.cid} ({cfg.name}): {L} layers generated and resident in {time.time() - t0:.1f}s")

    ws = layers[0].workspace(B, device=dev)
    y = torch.empty((L, B, cfg.d), dtype=torch.float32, device=dev)
    counts = torch.zeros((W + K, L, 2), dtype=torch.int32, device=dev)

    def step(t):
        for l in range(L):
            lay = layers[l]
            _abi.pi_ffn_layer(lay.pred, lay.ffn, xd[t, l], B, y[l], None, None, counts[t, l], ws)

    # ------------------------------------------------------------------ graph capture + timing
    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        step(0)
        torch.cuda.synchronize()
        if not args.no_graph:
            g_warm, g_timed = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_warm, stream=stream):
                for t in range(W):
                    step(t)
            with torch.cuda.graph(g_timed, stream=stream):
                for t in range(W, W + K):
                    step(t)
            torch.cuda.synchronize()
            g_warm.replay()
        else:
            for t in range(W):
                step(t)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        if not args.no_graph:
            g_timed.replay()
        else:
            for t in range(W, W + K):
                step(t)
        ev1.record(stream)
        torch.cuda.synchronize()
        elapsed_ms = ev0.elapsed_time(ev1)
    log(f"timed {K} steps: {elapsed_ms:.3f} ms")

    cnt = counts[W:].cpu().numpy()                              # [K][L][2]
    n_act = cnt[..., 0].astype(np.float64)
    n_pred = cnt[..., 1].astype(np.float64)

    # ------------------------------------------------------------------ bytes per step
    rb = cfg.row_bytes()
    in_rows = 2 if cfg.gated else 1
    pred_bytes = 2 * (cfg.r * cfg.d + cfg.f * cfg.r + cfg.f)
    act_bytes = n_act * (in_rows + 1) * rb                       # [K][L] predicted-active rows
    step_bytes = (pred_bytes * L + act_bytes.sum(axis=1))        # per step

    # ------------------------------------------------------------------ roofline pass (eager, HIP events)
    R = min(args.roofline_steps, K)
    seg = {"predict": 0.0, "compact": 0.0, "sparse_ffn": 0.0}
    touched_down = 0.0
    act_rows_rf = 0.0
    mask = torch.empty(cfg.f, dtype=torch.uint8, device=dev)
    idx = torch.empty(cfg.f, dtype=torch.int32, device=dev)
    cnt1 = torch.empty(2, dtype=torch.int32, device=dev)
    ws_p = torch.empty(_abi.pi_workspace_bytes(layers[0].pred, None, B), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(_abi.pi_workspace_bytes(None, layers[0].ffn, B), dtype=torch.uint8, device=dev)
    h_view = ws_f[: B * layers[0].n_slots * 4].view(torch.float32).view(B, layers[0].n_slots)
    with torch.cuda.stream(stream):
        evs = []
        for t in range(W, W + R):
            for l in range(L):
                lay = layers[l]
                e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                e[0].record(stream)
                _abi.pi_predict(lay.pred, xd[t, l], B, mask, None, ws_p)
                e[1].record(stream)
                _abi.pi_compact(mask, cfg.f, lay.slot_of, idx, cnt1)
                e[2].record(stream)
                _abi.pi_sparse_ffn(lay.ffn, xd[t, l], B, idx, cnt1, y[l], ws_f)
                e[3].record(stream)
                n = cnt1[0]
                nz = (h_view[:, :].narrow(1, 0, lay.n_slots) != 0).any(dim=0)
                k = torch.arange(lay.n_slots, device=dev) < n
                evs.append((e, (nz & k).sum(), n))
        torch.cuda.synchronize()
    for e, nz, n in evs:
        seg["predict"] += e[0].elapsed_time(e[1])
        seg["compact"] += e[1].elapsed_time(e[2])
        seg["sparse_ffn"] += e[2].elapsed_time(e[3])
        touched_down += float(nz)
        act_rows_rf += float(n)
    launches = R * L
    us = {k: v * 1000.0 / launches for k, v in seg.items()}     # per layer launch
    ffn_alg_bytes = act_rows_rf * in_rows * rb + touched_down * rb   # bytes the FFN kernels must read
    ffn_pred_bytes = act_rows_rf * (in_rows + 1) * rb
    ffn_gbs = ffn_alg_bytes / launches / (us["sparse_ffn"] * 1e-6) / 1e9
    pred_gbs = pred_bytes / (us["predict"] * 1e-6) / 1e9

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        budget = args.cpu_seconds
        done, spent, l = 0, 0.0, 0
        while spent < budget and done < 4 * L:
            host = synth.make_layer(cfg, l % L)
            x = x_all[W, l % L]
            s0 = time.perf_counter()
            oracle.ffn_layer(host, x, want_logits=False)
            spent += time.perf_counter() - s0
            done += 1
            l += 1
            del host
        per_layer = spent / done
        cpu = {"value": B / (per_layer * L), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{done} (layer, batch) evaluations of the full layer (predictor + mask + compaction + "
                         f"sparse FFN) at batch {B}, first token, layers 0..{min(done, L) - 1}; "
                         f"{spent:.1f}s, {per_layer * 1e3:.1f} ms per layer, scaled to a {L}-layer step"}

    ms_per_step = elapsed_ms / K
    tokens_per_s = B * K / (elapsed_ms / 1e3)
    step_gb = float(step_bytes.mean()) / 1e9
    out = {
        "metric": "sparse-FFN decode tokens/s (batch 1) + achieved HBM GB/s on active-row bytes",
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if cfg.wtype == synth.F16 else "q4_0",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {L} layers, d_model={cfg.d}, d_ffn={cfg.f}, predictor rank {cfg.r}, "
                        f"{'ReGLU' if cfg.gated else 'ReLU'}, {'fp16' if cfg.wtype == synth.F16 else 'Q4_0'} "
                        f"weights, batch {B}, Zipf firing at {cfg.density:.0%} target density"
                        + (f", hottest {cfg.hot_frac:.0%} resident" if cfg.hot_frac else ""),
            "global_batch": B, "layers": L, "d_model": cfg.d, "d_ffn": cfg.f, "rank": cfg.r,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "pi_sparse_ffn (k_sparse_up + k_sparse_down + k_reduce_y)",
            "achieved": round(ffn_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(ffn_gbs / PEAK_HBM_GBS, 4),
            "traffic": None,
        },
        "cpu_baseline": cpu,
        "detail": {
            "us_per_layer": round(ms_per_step * 1000.0 / L, 3),
            "step_gb_algorithmic": round(step_gb, 4),
            "step_gbs": round(step_gb / (ms_per_step / 1e3), 1),
            "active_density": round(float(n_act.mean()) / cfg.f, 4),
            "predicted_density": round(float(n_pred.mean()) / cfg.f, 4),
            "covered_share": round(float(n_act.sum() / max(n_pred.sum(), 1)), 4),
            "eager_us_per_layer": {k: round(v, 3) for k, v in us.items()},
            "predict_gbs": round(pred_gbs, 1),
            "ffn_bytes_per_layer_touched": round(ffn_alg_bytes / launches),
            "ffn_bytes_per_layer_predicted": round(ffn_pred_bytes / launches),
            "down_rows_skipped_share": round(1.0 - touched_down / max(act_rows_rf, 1), 4),
        },
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
