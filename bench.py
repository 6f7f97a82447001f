"""Throughput of the dual-codebook quantization loop on one MI355X.

A step is one pass of the whole path over one synthetic decoder layer whose inputs are resident
in HBM: importance of every activation stream, quantile init of every matrix, `iters` x (batched
assign, batched refine) with bf16 tables on the last refine, the final assign, pack and dequant.

Metric (value): bf16 weight bytes quantized per second per assign+refine iteration,
2 * numel * iters / t_loop, with t_loop the HIP-event time of the loop region of a step.
roofline: the dominant of the two loop kernels (assign, refine); achieved = its algorithmic bytes
per launch / its mean launch duration (HIP events on the launch stream); traffic = its HBM bytes per
launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by a plain copy), or null
when that summary was taken on other kernel sources or on another workload.
cpu_baseline: the fp64 oracle, assign + refine on a sample matrix, timed on the host.
inference: after the timed steps, the decode GEMV over the packed layer and the AWQ pre-scale of
the layer, each against the HBM peak (outside the metric).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-cpu]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_assign_refine_llama8b_layer.json")


def algorithmic_bytes(numel, S):
    """Bytes one assign or one refine launch must move per weight: read W (2), write or read the
    4-bit codes (0.5) and the selectors (1/S)."""
    return numel * (2.0 + 0.5 + 1.0 / S)


def cpu_baseline(W, I, g, S, n, budget_s=15.0):
    """Oracle assign+refine iterations on one matrix (host copy), until about budget_s seconds."""
    import numpy as np

    from oracle import aaac_ref as ref

    W64 = W.float().cpu().numpy().astype(np.float64)
    I64 = I.cpu().numpy().astype(np.float64)
    T0, T1 = ref.init_tables(W64, g, n)
    its = 0
    t0 = time.perf_counter()
    while True:
        a = ref.assign(W64, I64, T0, T1, g, S)
        T0, T1 = ref.refine(W64, I64, a["codes"], a["sel"], T0, T1, g, S)
        its += 1
        el = time.perf_counter() - t0
        if el >= budget_s or its >= 50:
            break
    return {"value": round(2.0 * W64.size * its / el / 1e9, 6), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": "%d oracle assign+refine iterations (fp64 NumPy, one thread) on the "
                      "%dx%d matrix of the layer, %.1f s" % (its, W64.shape[0], W64.shape[1], el)}


def inference_side(L, torch, dev, stream, mats, codes, scales, bitmaps, tb16, Ws, Is, g, S, n,
                   reps=8):
    """The two entry points around the loop, timed on this layer after the quantization steps:
    the decode GEMV over every packed matrix in one launch (batch 1), with 512 MB read between
    launches so that the packed weights come from HBM and not from the 256 MB last-level cache,
    and the AWQ pre-scale of every matrix (read W, write W_scaled)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    Rs = [m.rows for m in mats]
    Cs = [m.cols for m in mats]
    xs = [torch.randn(1, C, device=dev, generator=gen).to(torch.bfloat16) for C in Cs]
    ys = [torch.empty(R, device=dev) for R in Rs]
    flush = torch.ones(1 << 27, dtype=torch.float32, device=dev)
    bms = None if S == g else bitmaps
    gemv_bytes = sum(R * C // 2 + 2 * (R * C // g) + ((R * C // S + 7) // 8 if S < g else 0)
                     + 2 * C + 4 * R for R, C in zip(Rs, Cs))
    ts = []
    for r in range(reps + 1):
        flush.sum()                    # reads 512 MB: evicts the packed layer with clean lines
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        L.aaac_gemv_batch(codes, scales, bms, tb16, Rs, Cs, g, S, n, xs, ys)
        e1.record(stream)
        torch.cuda.synchronize()
        if r:
            ts.append(e0.elapsed_time(e1))
    del flush
    gemv_ms = sorted(ts)[len(ts) // 2]
    a = [torch.exp(0.5 * torch.randn(C, device=dev, generator=gen)) for C in Cs]
    W_s = [torch.empty_like(W) for W in Ws]
    I_s = [torch.empty_like(I) for I in Is]
    ts = []
    for r in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i, W in enumerate(Ws):
            L.aaac_awq_prescale(W, a[i], W_s[i], Is[i], I_s[i])
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    awq_ms = min(ts)
    awq_bytes = sum(4 * R * C + 12 * C for R, C in zip(Rs, Cs))
    gb = gemv_bytes / (gemv_ms * 1e-3) / 1e9
    ab = awq_bytes / (awq_ms * 1e-3) / 1e9
    return {
        "gemv": {"workload": "decode GEMV, batch 1, every linear of the layer in one launch, "
                             "packed weights cold in HBM",
                 "us_per_launch": round(gemv_ms * 1e3, 2), "bytes_per_launch": gemv_bytes,
                 "achieved": round(gb, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(gb / HBM_PEAK_GBS, 4)},
        "awq_prescale": {"workload": "W diag(a) and I / a^2 for every linear of the layer, "
                                     "one launch per matrix",
                         "us_per_layer": round(awq_ms * 1e3, 2), "bytes": awq_bytes,
                         "achieved": round(ab, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ab / HBM_PEAK_GBS, 4)},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--one-stream", action="store_true",
                    help="run init after importance on one stream (for per-kernel profiles)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this implementation has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import post_weight_quantization_06_amd as pkg
    from post_weight_quantization_06_amd import pmc_traffic
    from synth import layers as syn

    L = pkg._lib
    L.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = syn.config(args.config)
    if cfg.layers != 1:
        raise SystemExit("bench.py times one resident layer; config %d streams %d layers"
                         % (args.config, cfg.layers))
    g, S, n, iters = cfg.g, cfg.S, cfg.n, cfg.iters
    mats = cfg.matrices
    print("[bench] generating %s" % cfg.name, file=sys.stderr, flush=True)
    Ws = [syn.make_weight(m.rows, m.cols, syn.seed_for(cfg.cfg_id, 0, m.tensor_id), dev)
          for m in mats]
    streams = cfg.x_streams()
    Xs = {xid: syn.make_activations(cfg.tokens, K, syn.seed_for(cfg.cfg_id, 0, xid), dev)
          for xid, K in streams}
    torch.cuda.synchronize()
    numel = sum(m.numel for m in mats)
    Rs = [m.rows for m in mats]
    Cs = [m.cols for m in mats]

    # buffers and workspaces (allocated once)
    acc = {xid: torch.zeros(K, dtype=torch.float64, device=dev) for xid, K in streams}
    Iv = {xid: torch.empty(K, dtype=torch.float32, device=dev) for xid, K in streams}
    ws_imp = {xid: L.workspace(L.workspace_bytes(L.OP_IMPORTANCE, cfg.tokens, K), dev)
              for xid, K in streams}
    ws_init = L.workspace(L.batch_workspace_bytes(L.OP_INIT, Rs, Cs, g, 8, n), dev)
    ws_r = L.workspace(L.batch_workspace_bytes(L.OP_REFINE, Rs, Cs, g, S, n), dev)
    Is = [Iv[m.x_id] for m in mats]
    tabs = [torch.empty(2 * n, dtype=torch.float32, device=dev) for _ in mats]
    codes = [torch.empty(m.numel // 2, dtype=torch.uint8, device=dev) for m in mats]
    sels = [torch.empty(m.numel // S, dtype=torch.uint8, device=dev) for m in mats]
    scales = [torch.empty(m.numel // g, dtype=torch.int16, device=dev) for m in mats]
    bitmaps = [torch.empty((m.numel // S + 7) // 8, dtype=torch.uint8, device=dev)
               if S < g else None for m in mats]
    tb16 = [torch.empty(2 * n, dtype=torch.int16, device=dev) for _ in mats]
    W_hat = [torch.empty_like(W) for W in Ws]
    stream = torch.cuda.current_stream()

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    # init reads only W and importance only X, so init runs on a second stream (default priority,
    # like every stream here) beside importance; the loop waits for both
    side = stream if args.one_stream else torch.cuda.Stream(device=dev)

    def step(idx):
        # HIP events around the launches of two of the iterations (rotating with the step index)
        # time assign and refine live; an event record between every pair of launches would add
        # about 110 us to the 3.1 ms loop
        marks = {"a": [], "r": []}
        probe = set() if idx < 0 else {idx % iters, (idx + iters // 2) % iters}
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            L.aaac_init_quantiles_batch(Ws, g, n, tabs, ws_init)
        for xid, K in streams:
            acc[xid].zero_()
            L.aaac_importance(Xs[xid], acc[xid], Iv[xid], ws_imp[xid])
        stream.wait_stream(side)
        loop0 = ev()
        for it in range(iters):
            flags = L.REFINE_ROUND_BF16 if it == iters - 1 else 0
            if it not in probe:
                L.aaac_assign_batch(Ws, g, S, n, Is, tabs, codes, sels)
                L.aaac_refine_batch(Ws, g, S, n, Is, codes, sels, tabs, flags, ws_r)
                continue
            e0 = ev()
            L.aaac_assign_batch(Ws, g, S, n, Is, tabs, codes, sels)
            e1 = ev()
            L.aaac_refine_batch(Ws, g, S, n, Is, codes, sels, tabs, flags, ws_r)
            e2 = ev()
            marks["a"].append((e0, e1))
            marks["r"].append((e1, e2))
        loop1 = ev()
        L.aaac_assign_batch(Ws, g, S, n, Is, tabs, codes, sels)
        bms = bitmaps if S < g else None
        L.aaac_pack_batch(Ws, g, S, n, sels, tabs, scales, bms, tb16)
        L.aaac_dequant_batch(codes, scales, bms, tb16, Rs, Cs, g, S, n, W_hat)
        return loop0, loop1, marks

    # one plain device-to-device copy of 1 GiB, outside the timed region: the reference launch that
    # HBM byte counters (FETCH_SIZE / WRITE_SIZE) are scaled by
    calib_src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst
    for _ in range(args.warmup):
        step(-1)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    t_start = time.perf_counter()
    s0 = ev()
    recs = [step(i) for i in range(args.steps)]
    s1 = ev()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = s0.elapsed_time(s1) / args.steps
    loop_ms = sum(a.elapsed_time(b) for a, b, _ in recs) / args.steps
    a_ms = [x.elapsed_time(y) for _, _, m in recs for x, y in m["a"]]
    r_ms = [x.elapsed_time(y) for _, _, m in recs for x, y in m["r"]]
    a_avg = sum(a_ms) / len(a_ms)
    r_avg = sum(r_ms) / len(r_ms)
    bytes_launch = algorithmic_bytes(numel, S)
    dom, dom_ms = ("assign", a_avg) if a_avg >= r_avg else ("refine", r_avg)
    achieved = bytes_launch / (dom_ms * 1e-3) / 1e9
    value = 2.0 * numel * iters / (loop_ms * 1e-3) / 1e9
    print("[bench] step %.3f ms, loop %.3f ms, assign %.1f us (%.0f GB/s), refine %.1f us "
          "(%.0f GB/s), wall %.2f s" % (step_ms, loop_ms, a_avg * 1e3,
                                        bytes_launch / a_avg / 1e6, r_avg * 1e3,
                                        bytes_launch / r_avg / 1e6, wall),
          file=sys.stderr, flush=True)
    traffic = None
    if args.config == 2:
        t = pmc_traffic.load_traffic(TRAFFIC_SUMMARY, dom)
        traffic = None if t is None else int(round(t))
    inference = inference_side(L, torch, dev, stream, mats, codes, scales, bitmaps, tb16, Ws, Is,
                               g, S, n)
    print("[bench] gemv %.1f us (%.0f GB/s), awq prescale %.1f us (%.0f GB/s)" % (
        inference["gemv"]["us_per_launch"], inference["gemv"]["achieved"],
        inference["awq_prescale"]["us_per_layer"], inference["awq_prescale"]["achieved"]),
        file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu:
        k = min(range(len(mats)), key=lambda i: mats[i].numel)
        print("[bench] cpu baseline on %s" % mats[k].name, file=sys.stderr, flush=True)
        cpu = cpu_baseline(Ws[k], Is[k], g, S, n, args.cpu_budget)
    out = {
        "metric": "bf16 weights quantized/sec per assign+refine iter (GB/s) and % of HBM peak",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "matrices": [[m.rows, m.cols] for m in mats],
                   "numel": numel, "g": g, "S": S, "n": n, "iters": iters,
                   "calib_tokens": cfg.tokens},
        "loop_ms_per_step": round(loop_ms, 4),
        "assign_us": round(a_avg * 1e3, 2),
        "refine_us": round(r_avg * 1e3, 2),
        "hbm_frac_assign": round(bytes_launch / (a_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "hbm_frac_refine": round(bytes_launch / (r_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "bytes per launch",
                     "algorithmic_bytes": int(round(bytes_launch)),
                     "launches_timed": len(a_ms) if dom == "assign" else len(r_ms)},
        "cpu_baseline": cpu,
        "inference": inference,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
