"""Throughput of the dual-codebook quantization loop on one MI355X.

A step is one pass of the whole path over one synthetic workload whose inputs are resident in HBM.
Per decoder layer: importance of every activation stream, quantile init of every matrix (beside the
importance, on a second stream), `iters` x (batched assign with its error totals, batched refine)
with bf16 tables on the last refine, the final assign, pack and dequant. The default workload is the
32B-shaped model: 64 layers, every layer's weights resident (62.4 GB of bf16), quantized one layer
after another.

Metric (value): bf16 weight bytes quantized per second per assign+refine iteration,
2 * numel * iters / t_loop, with t_loop the HIP-event time of the loop regions of a step (summed
over the layers).
roofline: the dominant of the two loop kernels (assign, refine); achieved = its algorithmic bytes
per launch / its mean launch duration (HIP events on the launch stream); traffic = its HBM bytes per
launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of this workload (scaled by a
plain copy), or null when that summary was taken on other kernel sources.
cpu_baseline: the fp64 oracle (assign + refine iterations) on a sample of the workload's matrices,
one single-threaded worker process per matrix, timed on the host.
inference: after the timed steps, the decode GEMV over one packed layer and the AWQ pre-scale of
that layer, each against the HBM peak (outside the metric).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5] [--no-cpu]
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
TRAFFIC_SUMMARY = {
    2: os.path.join(ROOT, "profiles", "hbm_traffic_assign_refine_llama8b_layer.json"),
    5: os.path.join(ROOT, "profiles", "hbm_traffic_assign_refine_32b_model.json"),
}
TRAFFIC_SUMMARY_FUSED = {
    5: os.path.join(ROOT, "profiles", "hbm_traffic_assign_refine_32b_model_fused.json"),
}


def algorithmic_bytes(numel, S):
    """Bytes one assign or one refine launch must move per weight: read W (2), write or read the
    4-bit codes (0.5) and the selectors (1/S)."""
    return numel * (2.0 + 0.5 + 1.0 / S)


# ------------------------------------------------------------------------------------------------
# CPU baseline: the oracle in worker processes (test infrastructure, timed beside the GPU)
# ------------------------------------------------------------------------------------------------

def _oracle_worker(args):
    """One worker: oracle init, then assign + refine iterations on one matrix until the budget is
    spent. Runs in a fresh process with one BLAS/OpenMP thread."""
    bits, R, C, I32, g, S, n, budget = args
    import numpy as np

    from oracle import aaac_ref as ref

    W64 = ref.bits_to_float(np.frombuffer(bits, dtype=np.uint16).reshape(R, C))
    I64 = np.frombuffer(I32, dtype=np.float32).astype(np.float64)
    T0, T1 = ref.init_tables(W64, g, n)
    its = 0
    t0 = time.perf_counter()
    while True:
        a = ref.assign(W64, I64, T0, T1, g, S)
        T0, T1 = ref.refine(W64, I64, a["codes"], a["sel"], T0, T1, g, S)
        its += 1
        el = time.perf_counter() - t0
        if el >= budget:
            break
    return its, el, R * C


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _worker_ready(_):
    import numpy  # noqa: F401  (loaded before the GPU is touched in the parent)

    from oracle import aaac_ref  # noqa: F401
    return os.getpid()


def start_cpu_pool(workers):
    """Worker processes for the CPU baseline, started before the parent touches the GPU (each
    child is a fresh interpreter with one BLAS/OpenMP thread)."""
    import concurrent.futures
    import multiprocessing as mp

    env_keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in env_keys}
    for k in env_keys:
        os.environ[k] = "1"
    try:
        ex = concurrent.futures.ProcessPoolExecutor(max_workers=workers,
                                                    mp_context=mp.get_context("spawn"))
        pids = set(ex.map(_worker_ready, range(4 * workers)))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return ex, len(pids)


def cpu_baseline(pool, jobs, g, S, n, budget_s, workers):
    """jobs: list of (name, W bf16 tensor, I fp32 tensor), one per worker process of pool; the rate
    is the summed weight bytes per iteration over the longest worker's time."""
    import numpy as np
    import torch

    payload = []
    for _, W, I in jobs:
        bits = W.view(torch.int16).cpu().numpy().view(np.uint16).tobytes()
        payload.append((bits, W.shape[0], W.shape[1],
                        I.float().cpu().numpy().tobytes(), g, S, n, budget_s))
    t0 = time.perf_counter()
    res = list(pool.map(_oracle_worker, payload))
    wall = time.perf_counter() - t0
    weight_bytes = sum(2.0 * numel * its for its, _, numel in res)
    busy = max(el for _, el, _ in res)
    names = sorted({name for name, _, _ in jobs})
    shapes = sorted({"%dx%d" % tuple(W.shape) for _, W, _ in jobs})
    return {"value": round(weight_bytes / busy / 1e9, 6), "unit": "GB/s",
            "cores": workers, "kind": "oracle",
            "sample": "%d matrices (%s, %s) of the workload, each in its own single-threaded "
                      "worker process (fp64 NumPy oracle: init, then assign + refine iterations "
                      "for about %.0f s; %d iterations in all; pool wall %.1f s)"
                      % (len(jobs), ", ".join(names), "/".join(shapes), budget_s,
                         sum(its for its, _, _ in res), wall),
            "host": {"cpu": _cpu_model(), "os_cpu_count": os.cpu_count(),
                     "workers": workers}}


def _env_info(torch, dev):
    """The GPU, its architecture and the software versions the numbers were taken with."""
    rocm = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as f:
                rocm = f.read().strip()
            break
        except OSError:
            pass
    props = torch.cuda.get_device_properties(dev)
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", None),
            "cus": props.multi_processor_count, "rocm": rocm, "hip": torch.version.hip,
            "torch": torch.__version__}


# ------------------------------------------------------------------------------------------------
# Inference side (outside the metric)
# ------------------------------------------------------------------------------------------------

def inference_side(L, torch, dev, stream, shapes, buf, Ws, Is, g, S, n, reps=8):
    """The two entry points around the loop, timed on one layer after the quantization steps:
    the decode GEMV over every packed matrix of the layer in one launch (batch 1), with 512 MB read
    between launches so that the packed weights come from HBM and not from the 256 MB last-level
    cache, and the AWQ pre-scale of every matrix (read W, write W_scaled)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    Rs = [R for R, _ in shapes]
    Cs = [C for _, C in shapes]
    xs = [torch.randn(1, C, device=dev, generator=gen).to(torch.bfloat16) for C in Cs]
    ys = [torch.empty(R, device=dev) for R in Rs]
    flush = torch.ones(1 << 27, dtype=torch.float32, device=dev)
    bms = None if S == g else buf.bitmaps
    gemv_bytes = sum(R * C // 2 + 2 * (R * C // g) + ((R * C // S + 7) // 8 if S < g else 0)
                     + 2 * C + 4 * R for R, C in zip(Rs, Cs))
    ts = []
    for r in range(reps + 1):
        flush.sum()                    # reads 512 MB: evicts the packed layer with clean lines
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        L.aaac_gemv_batch(buf.codes, buf.scales, bms, buf.tables_bf16, Rs, Cs, g, S, n, xs, ys)
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
        "gemv": {"workload": "decode GEMV, batch 1, every linear of one layer in one launch, "
                             "packed weights cold in HBM",
                 "us_per_launch": round(gemv_ms * 1e3, 2), "bytes_per_launch": gemv_bytes,
                 "achieved": round(gb, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(gb / HBM_PEAK_GBS, 4)},
        "awq_prescale": {"workload": "W diag(a) and I / a^2 for every linear of one layer, "
                                     "one launch per matrix",
                         "us_per_layer": round(awq_ms * 1e3, 2), "bytes": awq_bytes,
                         "achieved": round(ab, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ab / HBM_PEAK_GBS, 4)},
    }


# ------------------------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-inference", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="oracle worker processes (capped by the host's CPU count)")
    ap.add_argument("--fused", action="store_true",
                    help="run each iteration as one aaac_assign_refine_batch launch (bitwise the "
                         "same results) instead of the assign and refine launches")
    ap.add_argument("--one-stream", action="store_true",
                    help="run init after importance on one stream (for per-kernel profiles)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this implementation has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    pool = None
    if not args.no_cpu:
        pool, started = start_cpu_pool(max(1, min(args.cpu_workers, os.cpu_count() or 1)))
        print("[bench] %d oracle worker processes started" % started, file=sys.stderr,
              flush=True)

    import torch

    import post_weight_quantization_06_amd as pkg
    from post_weight_quantization_06_amd import pmc_traffic
    from synth import layers as syn

    L = pkg._lib
    L.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = syn.config(args.config)
    g, S, n, iters = cfg.g, cfg.S, cfg.n, cfg.iters
    mats = cfg.matrices
    nl = cfg.layers
    shapes = [(m.rows, m.cols) for m in mats]
    print("[bench] generating %s (%d layer%s)" % (cfg.name, nl, "s" if nl > 1 else ""),
          file=sys.stderr, flush=True)
    Ws = [[syn.make_weight(m.rows, m.cols, syn.seed_for(cfg.cfg_id, l, m.tensor_id), dev)
           for m in mats] for l in range(nl)]
    # the activation streams of one layer, resident; every layer of a multi-layer model reads this
    # one set (each layer's own activations would come from running the previous layers on
    # calibration text; synthesizing 90 GB per layer is input generation, not the path)
    streams = cfg.x_streams()
    Xs = {xid: syn.make_activations(cfg.tokens, K, syn.seed_for(cfg.cfg_id, 0, xid), dev)
          for xid, K in streams}
    torch.cuda.synchronize()
    numel_layer = sum(m.numel for m in mats)
    numel = numel_layer * nl
    Rs = [R for R, _ in shapes]
    Cs = [C for _, C in shapes]
    print("[bench] %d weights resident, %.1f GB of activations" % (
        numel, sum(X.numel() * 4 for X in Xs.values()) / 1e9), file=sys.stderr, flush=True)

    # buffers and workspaces (allocated once)
    wsp = pkg.Workspaces(dev)
    acc = {xid: torch.zeros(K, dtype=torch.float64, device=dev) for xid, K in streams}
    Iv = {xid: torch.empty(K, dtype=torch.float32, device=dev) for xid, K in streams}
    ws_init = L.workspace(L.batch_workspace_bytes(L.OP_INIT, Rs, Cs, g, 8, n), dev)
    Is = [Iv[m.x_id] for m in mats]
    bufs = [pkg.LayerBuffers(shapes, g, S, n, iters, dev) for _ in range(nl)]
    W_hat = [torch.empty(R, C, dtype=torch.bfloat16, device=dev) for R, C in shapes]
    stream = torch.cuda.current_stream()

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    class Timing(pkg.Probe):
        """HIP events around the launches of two of the iterations of every layer (rotating with
        the layer and step), and around each layer's whole loop."""

        def __init__(self, probe_its):
            self.probe_its = probe_its
            self.a, self.r, self.loops = [], [], []
            self._e = None

        def loop_begin(self):
            self._l0 = ev()

        def loop_end(self):
            self.loops.append((self._l0, ev()))

        def before_assign(self, it):
            self._e = ev() if it in self.probe_its else None

        def before_refine(self, it):
            if self._e is not None:
                e1 = ev()
                self.a.append((self._e, e1))
                self._e = e1

        def after_refine(self, it):
            if self._e is not None:
                self.r.append((self._e, ev()))
                self._e = None

    # init reads only W and importance only X, so init runs on a second stream (default priority,
    # like every stream here) beside importance; the loop waits for both
    side = stream if args.one_stream else torch.cuda.Stream(device=dev)

    def step(idx):
        timing = None
        for l in range(nl):
            probe = (set() if idx < 0 else
                     {(idx + l) % iters, (idx + l + iters // 2) % iters})
            t = Timing(probe)
            buf = bufs[l]
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                L.aaac_init_quantiles_batch(Ws[l], g, n, buf.tables, ws_init)
            for xid, K in streams:
                acc[xid].zero_()
                L.aaac_importance(Xs[xid], acc[xid], Iv[xid],
                                  wsp.get(("importance", xid), L.workspace_bytes(
                                      L.OP_IMPORTANCE, Xs[xid].shape[0], K)))
            stream.wait_stream(side)
            pkg.run_loop(Ws[l], Is, buf, wsp, init=False, probe=t, fused=args.fused)
            L.aaac_dequant_batch(buf.codes, buf.scales, buf.bitmaps, buf.tables_bf16, Rs, Cs,
                                 g, S, n, W_hat)
            if timing is None:
                timing = t
            else:
                timing.a += t.a
                timing.r += t.r
                timing.loops += t.loops
        return timing

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
    recs = []
    for i in range(args.steps):
        recs.append(step(i))
        if nl > 1:
            print("[bench] step %d enqueued" % i, file=sys.stderr, flush=True)
    s1 = ev()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = s0.elapsed_time(s1) / args.steps
    loop_ms = sum(a.elapsed_time(b) for t in recs for a, b in t.loops) / args.steps
    a_ms = [x.elapsed_time(y) for t in recs for x, y in t.a]
    r_ms = [x.elapsed_time(y) for t in recs for x, y in t.r]
    a_avg = sum(a_ms) / len(a_ms)
    r_avg = sum(r_ms) / len(r_ms)
    # one launch reads W and writes the codes and selectors (the fused launch does no more)
    bytes_launch = algorithmic_bytes(numel_layer, S)
    if args.fused:
        dom, dom_ms = "fused", a_avg
    else:
        dom, dom_ms = ("assign", a_avg) if a_avg >= r_avg else ("refine", r_avg)
    achieved = bytes_launch / (dom_ms * 1e-3) / 1e9
    value = 2.0 * numel * iters / (loop_ms * 1e-3) / 1e9
    if args.fused:
        print("[bench] step %.3f ms, loop %.3f ms, fused %.1f us (%.0f GB/s), wall %.2f s" % (
            step_ms, loop_ms, a_avg * 1e3, bytes_launch / a_avg / 1e6, wall),
            file=sys.stderr, flush=True)
    else:
        print("[bench] step %.3f ms, loop %.3f ms, assign %.1f us (%.0f GB/s), refine %.1f us "
              "(%.0f GB/s), wall %.2f s" % (step_ms, loop_ms, a_avg * 1e3,
                                            bytes_launch / a_avg / 1e6, r_avg * 1e3,
                                            bytes_launch / r_avg / 1e6, wall),
              file=sys.stderr, flush=True)
    # the error totals of the last step: non-increasing over the iterations of every matrix
    for l in range(nl):
        pkg.check_history(bufs[l].err, w2=bufs[l].w2)
    last = bufs[nl - 1].err[:, 0].cpu().tolist()
    print("[bench] error history, last layer, first matrix: %s" % ", ".join(
        "%.6g" % x for x in last), file=sys.stderr, flush=True)
    traffic = None
    summaries = TRAFFIC_SUMMARY_FUSED if args.fused else TRAFFIC_SUMMARY
    if args.config in summaries:
        t = pmc_traffic.load_traffic(summaries[args.config], dom)
        traffic = None if t is None else int(round(t))
    inference = None
    if not args.no_inference:
        inference = inference_side(L, torch, dev, stream, shapes, bufs[0], Ws[0], Is, g, S, n)
        print("[bench] gemv %.1f us (%.0f GB/s), awq prescale %.1f us (%.0f GB/s)" % (
            inference["gemv"]["us_per_launch"], inference["gemv"]["achieved"],
            inference["awq_prescale"]["us_per_layer"], inference["awq_prescale"]["achieved"]),
            file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu:
        # the two smallest matrices (by size) of evenly spaced layers, one per worker
        workers = max(1, min(args.cpu_workers, os.cpu_count() or 1))
        order = sorted(range(len(mats)), key=lambda i: mats[i].numel)[:2]
        nsample = max(1, workers // len(order))
        layers = sorted({round(k * (nl - 1) / max(1, nsample - 1)) for k in range(nsample)})
        jobs = [(mats[i].name, Ws[l][i], Is[i]) for l in layers for i in order][:workers]
        print("[bench] cpu baseline: %d oracle workers" % len(jobs), file=sys.stderr, flush=True)
        cpu = cpu_baseline(pool, jobs, g, S, n, args.cpu_budget, len(jobs))
        cpu["sample"] += "; layers %s" % layers
        pool.shutdown()
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
        "config": {"workload": cfg.name, "layers": nl, "matrices": [list(s) for s in shapes],
                   "numel": numel, "g": g, "S": S, "n": n, "iters": iters,
                   "calib_tokens": cfg.tokens},
        "loop_ms_per_step": round(loop_ms, 4),
        "iteration": "one fused launch" if args.fused else "assign and refine launches",
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "bytes per launch",
                     "algorithmic_bytes": int(round(bytes_launch)),
                     "launches_timed": len(r_ms) if dom == "refine" else len(a_ms)},
        "cpu_baseline": cpu,
        "inference": inference,
        "env": _env_info(torch, dev),
    }
    if args.fused:
        out["fused_us"] = round(a_avg * 1e3, 2)
        out["hbm_frac_fused"] = round(bytes_launch / (a_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    else:
        out["assign_us"] = round(a_avg * 1e3, 2)
        out["refine_us"] = round(r_avg * 1e3, 2)
        out["hbm_frac_assign"] = round(bytes_launch / (a_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        out["hbm_frac_refine"] = round(bytes_launch / (r_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
