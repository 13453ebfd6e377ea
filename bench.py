#!/usr/bin/env python3
"""Decode-step benchmark of the predictor-gated sparse FFN stack on one MI355X.

A step is one token (or one batch of B tokens) through every layer of the stack: per layer the
predictor GEMVs, the firing mask and its compaction, and the sparse FFN over the active neurons
(pi_ffn_layer), with each (layer, token) fed its own seeded input vector.  Inputs and weights
are resident in HBM before timing starts.  W warmup steps and K timed steps are replayed from
HIP graphs captured on one stream; the timed region is bracketed by device synchronizations.

Printed: one JSON line with tokens/s, ms per step, per-layer microseconds, the roofline of the
step's dominant kernel on the bytes it reads (HIP events on the launch stream around a graph of
its launches), and
the CPU oracle's rate on a bounded sample of the same workload.
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


def measured_traffic(workload: str, kernel_prefix: str):
    """HBM bytes per launch (read + written) of the kernel whose name starts with kernel_prefix, from the
    counter summary in profiles/ for this workload -- None when there is none or the sources changed."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("sources_sha256") != kernel_sources_sha256():
        return None
    for name, v in rec.get("kernels", {}).items():
        if name.startswith(kernel_prefix):
            return int(v["read_bytes"]) + int(v["write_bytes"])
    return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128, help="timed decode steps (tokens per sequence)")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", type=int, default=2, help="layer-stack configuration id (1-5)")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--layers", type=int, default=0, help="use only the first N layers (0 = all)")
    ap.add_argument("--roofline-steps", type=int, default=16, help="tokens whose launches the roofline pass times")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph replay")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the measurement, run one device-to-device copy of this many MiB (a kernel of "
                         "known traffic, for scaling hardware byte counters)")
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

    def step(t):
        for l in range(L):
            lay = layers[l]
            _abi.pi_ffn_layer(lay.pred, lay.ffn, xd[t, l], B, y[l], None, None, None, ws)

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
    status = _abi.workspace_status(ws)
    if status != 0:
        raise RuntimeError(f"workspace status {status}: a cross-workgroup wait timed out; results invalid")
    log(f"timed {K} steps: {elapsed_ms:.3f} ms")

    # ------------------------------------------------------------------ per-kernel legs (HIP events)
    # pi_ffn_layer is pi_predict_hidden (z = ReLU(P1 x), one kernel) followed by
    # pi_ffn_layer_from_hidden (logits, mask and the sparse FFN: one persistent kernel on path 1).
    # An eager pass runs both on R tokens x L layers, keeping every z and every index list, and
    # runs pi_sparse_ffn on each list (the sparse FFN alone, one kernel) to count the listed
    # neurons whose h is nonzero for some token.  Then the R*L launches of each entry point are
    # captured into a graph of their own and timed with HIP events on the launch stream around
    # its replay: elapsed / launches is the average launch duration, back to back as in the step.
    R = min(args.roofline_steps, K)
    N = R * L
    rb = cfg.row_bytes()
    in_rows = 2 if cfg.gated else 1
    pred_bytes = 2 * (cfg.r * cfg.d + cfg.f * cfg.r + cfg.f)
    path = _abi.pi_layer_path(layers[0].pred, layers[0].ffn, B)
    z_all = torch.empty((N, B, cfg.r), dtype=torch.float32, device=dev)
    masks = torch.empty((N, cfg.f), dtype=torch.uint8, device=dev)
    idx_all = torch.empty((N, cfg.f), dtype=torch.int32, device=dev)
    cnt_all = torch.empty((N, 2), dtype=torch.int32, device=dev)
    ws_f = torch.zeros(_abi.pi_workspace_bytes(None, layers[0].ffn, B), dtype=torch.uint8, device=dev)
    y_chk = torch.empty((B, cfg.d), dtype=torch.float32, device=dev)
    ns = layers[0].n_slots
    ar = torch.arange(ns, device=dev)
    cases = [(W + i // L, i % L) for i in range(N)]             # (token, layer) of launch i

    def run_hidden():
        for i, (t, l) in enumerate(cases):
            _abi.pi_predict_hidden(layers[l].pred, xd[t, l], B, z_all[i])

    def run_rest():
        for i, (t, l) in enumerate(cases):
            _abi.pi_ffn_layer_from_hidden(layers[l].pred, layers[l].ffn, xd[t, l], B, z_all[i], y_chk, None, None,
                                          None, ws)

    def run_sparse():
        for i, (t, l) in enumerate(cases):
            _abi.pi_sparse_ffn(layers[l].ffn, xd[t, l], B, idx_all[i], cnt_all[i], y_chk, ws_f)

    with torch.cuda.stream(stream):
        run_hidden()
        for i, (t, l) in enumerate(cases):
            _abi.pi_ffn_layer_from_hidden(layers[l].pred, layers[l].ffn, xd[t, l], B, z_all[i], y_chk, masks[i],
                                          idx_all[i], cnt_all[i], ws)
        live = []
        for i, (t, l) in enumerate(cases):
            _abi.pi_sparse_ffn(layers[l].ffn, xd[t, l], B, idx_all[i], cnt_all[i], y_chk, ws_f)
            h, ok = _abi.sparse_ffn_h(layers[l].ffn, B, ws_f, ns)
            live.append(((h != 0).any(dim=0) & ok & (ar < cnt_all[i, 0])).sum())
        torch.cuda.synchronize()
        n_live = torch.stack(live).cpu().numpy().astype(np.float64)
        cnt_host = cnt_all.cpu().numpy().astype(np.float64)
        leg_us = {}
        for name, fn in (("hidden", run_hidden), ("rest", run_rest), ("sparse_ffn", run_sparse)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                fn()
            g.replay()                                          # warm
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            leg_us[name] = e0.elapsed_time(e1) * 1000.0 / N
            del g
    for w in (ws, ws_f):
        if _abi.workspace_status(w) != 0:
            raise RuntimeError("workspace status nonzero: a cross-workgroup wait timed out")
    n_act, n_pred = cnt_host[:, 0], cnt_host[:, 1]
    vec_bytes = B * cfg.d * (2 + 4) + 2 * cfg.d                  # x in, y out, b_down
    slot_bytes = 4 * cfg.f if layers[0].slot_of is not None else 0
    # sparse FFN alone: the persistent kernel and the MFMA form read every listed row (the former's
    # down-row loads go out before h is known); the GEMV two-kernel form skips down rows whose h is
    # zero for every token
    _, h_kind = _abi.pi_sparse_ffn_h_offset(layers[0].ffn, B)
    n_read_down = n_act if h_kind in (1, 3) else n_live
    ffn_touched = n_act * in_rows * rb + n_read_down * rb + 8 * n_act + vec_bytes
    ffn_predicted = n_act * (in_rows + 1) * rb + 8 * n_act + vec_bytes
    # the rest of the layer on path 1 (one kernel): P2 and c, z, every listed row in and down
    rest_bytes = 2 * cfg.f * cfg.r + 2 * cfg.f + 4 * B * cfg.r + slot_bytes + n_act * (in_rows + 1) * rb + vec_bytes
    hidden_bytes = 2 * cfg.r * cfg.d + 2 * B * cfg.d + 4 * B * cfg.r
    gname = "true" if cfg.gated else "false"
    wname = 1 if cfg.wtype == synth.F16 else 2
    if path == 1:
        roof_kernel = ("k_layer_tail (pi_ffn_layer_from_hidden: predictor logits and mask, gathered up/gate rows "
                       "with ReLU/ReGLU, active rows of W_down^T)")
        roof_bytes, roof_us = float(rest_bytes.mean()), leg_us["rest"]
        roof_prefix = f"void pik::k_layer_tail<{B}, {gname}, {wname},"
    else:
        roof_kernel = "k_sparse_ffn (pi_sparse_ffn: gathered up/gate rows with ReLU/ReGLU + active rows of W_down^T)"
        roof_bytes, roof_us = float(ffn_touched.mean()), leg_us["sparse_ffn"]
        roof_prefix = f"void pik::k_sparse_ffn<{B}, {gname}, {wname}>"
    workload_tag = f"{cfg.name}_b{B}"
    roof_traffic = measured_traffic(workload_tag, roof_prefix) if L == cfg.layers else None
    roof_gbs = roof_bytes / (roof_us * 1e-6) / 1e9
    step_bytes = (pred_bytes + float(ffn_touched.mean())) * L
    # ------------------------------------------------------------------ host half (placement stacks)
    # With a placement, the predicted neurons that are not resident are the host's share of the
    # hybrid split (pi_cold_ffn_host over the cold rows in host memory).  Timed here on the masks
    # the device produced, for the first layers of the stack.
    cold = None
    if layers[0].slot_of is not None:
        import synth as _s
        n_lay = min(L, 2)
        masks_h = masks.cpu().numpy()
        hosts = []
        for l in range(n_lay):
            _, _, _, freq = _s.make_predictor(cfg, l)
            cold_ids = np.setdiff1d(np.arange(cfg.f, dtype=np.int32), _s.hot_set(freq, cfg.n_hot()))
            w_in_c, w_dn_c, b_up_c, _ = _s.make_ffn(cfg, l, cold_ids)
            slot_c = np.full(cfg.f, -1, np.int32)
            slot_c[cold_ids] = np.arange(cold_ids.size, dtype=np.int32)
            hosts.append(_abi.HostFFN(w_in_c, w_dn_c, d_model=cfg.d, d_ffn=cfg.f, gated=cfg.gated, wtype=cfg.wtype,
                                      slot_of=slot_c, b_up=b_up_c))
        ws_h = np.zeros(_abi.pi_cold_workspace_bytes(hosts[0], B), np.uint8)
        y_h = np.empty((B, cfg.d), np.float32)
        # every host thread, and half of them (hosts that expose two threads per core often run this
        # memory-bound loop faster on one per core); the faster is reported, with its count
        best = None
        for nthr in sorted({_s.num_threads(), max(1, _s.num_threads() // 2)}):
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
        # the hybrid layer end to end, as the method runs it (device over the resident neurons,
        # host over the rest, y's added), with the layer's dependencies kept in order: device
        # layer -> mask to pinned host memory -> host half -> host y to the device -> added to y
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
                    _abi.pi_ffn_layer(layers[l].pred, layers[l].ffn, xd[t, l], B, y_dev, m_dev, None, None, ws)
                    mask_pin.copy_(m_dev, non_blocking=True)
                    stream.synchronize()
                    _abi.pi_cold_ffn_host(hosts[l], np.ascontiguousarray(x_all[t, l]), B, mask_pin.numpy(),
                                          ycold_pin.numpy(), ws_h, nthr)
                    yc_dev.copy_(ycold_pin, non_blocking=True)
                    y_dev.add_(yc_dev)
                    stream.synchronize()
                    if rep == 1:
                        hyb.append(time.perf_counter() - s0)
        del hosts
        cold_us = 1e6 * best[0]
        counts_c = best[2]
        cold = {"host_us_per_layer": round(cold_us, 2), "neurons_per_layer": round(float(np.mean(counts_c)), 1),
                "rows_mb_per_layer": round(float(np.mean(counts_c)) * (in_rows + 1) * rb / 1e6, 3),
                "threads": best[1], "calls": best[3],
                "hybrid_layer_us": round(1e6 * float(np.median(hyb)), 2),
                "device_only_layer_us": round(elapsed_ms * 1000.0 / (K * L), 2)}
    # ------------------------------------------------------------------ 16-token batches on MFMA
    # pi_sparse_ffn_wide over each layer's union of 16 tokens' predicted lists (the masks of the
    # eager pass above, ORed and compacted outside the timed region), x of those 16 tokens; one
    # graph of L launches, timed with HIP events on the launch stream.
    wide = None
    if B == 1 and R >= 16 and layers[0].slot_of is None:
        with torch.cuda.stream(stream):
            idx_w = torch.empty((L, cfg.f), dtype=torch.int32, device=dev)
            cnt_w = torch.empty((L, 2), dtype=torch.int32, device=dev)
            x_w = torch.empty((L, 16, cfg.d), dtype=torch.int16, device=dev)
            for l in range(L):
                sel = [i for i, (t, ll) in enumerate(cases) if ll == l][:16]
                union = masks[sel].amax(dim=0).contiguous()
                _abi.pi_compact(union, cfg.f, None, idx_w[l], cnt_w[l])
                x_w[l] = xd[[cases[i][0] for i in sel], l, 0]
            ws_w = torch.empty(_abi.pi_sparse_ffn_wide_workspace_bytes(layers[0].ffn, 16), dtype=torch.uint8,
                               device=dev)
            y_w = torch.empty((16, cfg.d), dtype=torch.float32, device=dev)

            def run_wide():
                for l in range(L):
                    _abi.pi_sparse_ffn_wide(layers[l].ffn, x_w[l], 16, idx_w[l], cnt_w[l], y_w, ws_w)

            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                run_wide()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            wide_us = e0.elapsed_time(e1) * 1000.0 / L
            del g
        n_w = cnt_w[:, 0].cpu().numpy().astype(np.float64)
        wide_bytes = float((n_w * (in_rows + 1) * rb + 4 * n_w).mean()) + 16 * cfg.d * (2 + 4) + 2 * cfg.d
        wide = {"batch": 16, "us_per_layer": round(wide_us, 3), "neurons_per_layer": round(float(n_w.mean()), 1),
                "algorithmic_bytes_per_layer": int(wide_bytes),
                "gb_per_s": round(wide_bytes / (wide_us * 1e-6) / 1e9, 1),
                "hbm_frac": round(wide_bytes / (wide_us * 1e-6) / 8e12, 4),
                "kernels": "k_wide_up + k_wide_down (pi_sparse_ffn_wide, MFMA 16x16x16 f16)"}
        log(f"16-token sparse FFN (MFMA): {wide_us:.1f} us/layer over {n_w.mean():.0f} neurons")

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        budget = args.cpu_seconds
        n_lay = min(L, 4)
        hosts = [synth.make_layer(cfg, l) for l in range(n_lay)]
        done, spent, t = 0, 0.0, 0
        while spent < budget:
            for l in range(n_lay):
                s0 = time.perf_counter()
                oracle.ffn_layer(hosts[l], x_all[t % (W + K), l], want_logits=False)
                spent += time.perf_counter() - s0
                done += 1
            t += 1
        del hosts
        per_layer = spent / done
        cpu = {"value": round(B / (per_layer * L), 3), "unit": "tokens/s", "cores": oracle.num_threads(),
               "kind": "oracle",
               "sample": f"{done} evaluations of the whole layer (predictor, mask, compaction, sparse FFN) at "
                         f"batch {B}: layers 0..{n_lay - 1} of the same stack, {t} token steps cycling over the "
                         f"{W + K} seeded inputs; {spent:.1f}s, {per_layer * 1e3:.2f} ms per layer, scaled to the "
                         f"{L}-layer step"}

    ms_per_step = elapsed_ms / K
    tokens_per_s = B * K / (elapsed_ms / 1e3)
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
            "kernel": roof_kernel,
            "achieved": round(roof_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(roof_gbs / PEAK_HBM_GBS, 4),
            "traffic": roof_traffic,
            "bytes_per_launch": round(roof_bytes),
            "launch_us": round(roof_us, 3),
            "launches": int(N),
        },
        "cpu_baseline": cpu,
        "detail": {
            "us_per_layer": round(ms_per_step * 1000.0 / L, 3),
            "layer_path": path,
            "graph_us_predict_hidden": round(leg_us["hidden"], 3),
            "graph_us_layer_from_hidden": round(leg_us["rest"], 3),
            "graph_us_sparse_ffn": round(leg_us["sparse_ffn"], 3),
            "bytes_predict_hidden": hidden_bytes,
            "bytes_layer_from_hidden": round(float(rest_bytes.mean())),
            "bytes_sparse_ffn_read": round(float(ffn_touched.mean())),
            "bytes_sparse_ffn_predicted_rows": round(float(ffn_predicted.mean())),
            "gbs_sparse_ffn": round(float(ffn_touched.mean()) / (leg_us["sparse_ffn"] * 1e-6) / 1e9, 1),
            "predictor_bytes": pred_bytes,
            "step_gb_algorithmic": round(step_bytes / 1e9, 4),
            "step_gbs": round(step_bytes / 1e9 / (ms_per_step / 1e3), 1),
            "active_density": round(float(n_act.mean()) / cfg.f, 4),
            "predicted_density": round(float(n_pred.mean()) / cfg.f, 4),
            "covered_share": round(float(n_act.sum() / max(n_pred.sum(), 1)), 4),
            "down_rows_zero_h_share": round(1.0 - float(n_live.sum()) / max(float(n_act.sum()), 1.0), 4),
            "cold_host": cold,
            "wide_b16": wide,
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
