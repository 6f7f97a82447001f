"""Text summaries of rocprofv3 runs of bench.py.

Turns the raw rocprofv3 output of the runs below (one counter group per run, all writing under
one folder RAW) into the short Markdown summaries kept in PROFILES, for one workload TAG
(`32b_model`: the 64-layer 32B-shaped model, bench.py --config 5; `llama8b_layer`: the 8B-shaped
decoder layer, --config 2; `32b_model_fused`: the 32B-shaped model with each iteration as one
fused launch, --config 5 --fused):

    rocprofv3 --kernel-trace --stats --output-format csv -d RAW/prof_TAG -o run -- \\
        python -u bench.py --config N [--fused] --steps 2 --warmup 1 --no-cpu --one-stream
    rocprofv3 --pmc FETCH_SIZE ... -d RAW/pmc_fetch_TAG ...  (bench.py --steps 1 --warmup 1)
    rocprofv3 --pmc WRITE_SIZE ... -d RAW/pmc_write_TAG ...
    rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU ... -d RAW/pmc_sq_TAG ...
    rocprofv3 --pmc SQ_WAIT_ANY SQ_WAIT_INST_LDS ... -d RAW/pmc_sq2_TAG ...
    rocprofv3 --pmc SQ_LDS_IDX_ACTIVE ... GRBM_GUI_ACTIVE -d RAW/pmc_lds_TAG ...
    rocprofv3 --pmc SQ_WAVE_CYCLES ... GRBM_GUI_ACTIVE -d RAW/pmc_gemv_TAG ...  (with the GEMV)
    python -m post_weight_quantization_06_amd.pmc_traffic FETCH.csv WRITE.csv TRAFFIC.json

Usage (from the repository root):

    python -m post_weight_quantization_06_amd.prof_summary RAW PROFILES [TAG]

Writes kernel_stats_TAG.md, hbm_traffic_assign_refine_TAG.{json,md} (the JSON from the two
counter runs) and sq_counters_assign_refine_TAG.md, whose command lines name RAW and PROFILES as
given. Missing counter runs are skipped.
"""

from __future__ import annotations

import collections
import csv
import json
import os
import sys

PEAK = 8e12

# workload tag -> (bench config, name, fused iterations)
WORKLOADS = {
    "32b_model": (5, "the 32B-shaped model (64 decoder layers, g=128, S=128, n=16, 10 iterations)",
                  False),
    "llama8b_layer": (2, "the 8B-shaped decoder layer (g=128, S=128, n=16, 10 iterations)", False),
    "32b_model_fused": (5, "the 32B-shaped model (64 decoder layers, g=128, S=128, n=16, 10 "
                           "iterations), each iteration one fused assign + accumulate launch",
                        True),
}
TRACE_STEPS = 3      # the trace command runs 1 warmup + 2 timed steps

SQ1 = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU SQ_WAVE_CYCLES SQ_BUSY_CYCLES "
       "SQ_WAIT_INST_ANY SQ_INSTS_VMEM_RD")
SQ2 = ("SQ_WAIT_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT "
       "SQ_ACTIVE_INST_ANY")
# how busy the CU's units are: the LDS (cycles it works on indexed operations, and cycles it stalls
# on bank or address conflicts) and the VALU, against the dispatch's active GPU cycles
SQ3 = ("SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_LDS_ADDR_CONFLICT SQ_LDS_DATA_FIFO_FULL "
       "SQ_ACTIVE_INST_VALU SQ_INSTS_LDS_ATOMIC GRBM_GUI_ACTIVE")
# the decode GEMV that bench.py runs after its steps: instruction counts and unit business
SQG = ("SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_INSTS_LDS SQ_WAIT_INST_LDS SQ_LDS_IDX_ACTIVE "
       "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE")
GEMV = "gemv_kernel<"
CUS = 256
XCDS = 8      # GRBM_GUI_ACTIVE comes back summed over the 8 XCDs, each counting the dispatch's cycles
WRITTEN_BY = ("Summary written by `python -m post_weight_quantization_06_amd.prof_summary {raw} "
              "{prof} {tag}` from the raw output of the commands below.\n")

# kernel families: (key, name fragment); the loop kernels of every template instance
ASSIGN = "aaac::assign_wide_kernel<"
REFINE = "aaac::refine_kernel<"
FUSED = "aaac::assign_refine_kernel<"


def loop_families(tag):
    """The loop kernels of a workload: (key, name fragment) for each family."""
    if WORKLOADS[tag][2]:
        return (("fused", FUSED),)
    return (("assign", ASSIGN + "0,"), ("refine", REFINE))


def _flags(tag):
    return " --fused" if WORKLOADS[tag][2] else ""


def workload(tag):
    """(config id, description, matrix shapes, layers, bytes of activations read per layer)."""
    from synth import layers as syn

    cfg_id, desc, _ = WORKLOADS[tag]
    cfg = syn.config(cfg_id)
    shapes = [(m.rows, m.cols) for m in cfg.matrices]
    x_bytes = 4 * cfg.tokens * sum(K for _, K in cfg.x_streams())
    return cfg_id, desc, shapes, cfg.layers, x_bytes


def trace_cmd(raw, tag, cfg_id):
    return ("rocprofv3 --kernel-trace --stats --output-format csv -d %s/prof_%s -o run -- "
            "python -u bench.py --config %d%s --steps 2 --warmup 1 --no-cpu --one-stream"
            % (raw, tag, cfg_id, _flags(tag)))


def pmc_cmd(counters, out, raw, cfg_id, tag):
    return ("rocprofv3 --pmc %s --output-format csv -d %s/%s -o run -- python -u bench.py "
            "--config %d%s --steps 1 --warmup 1 --no-cpu --no-inference --one-stream"
            % (counters, raw, out, cfg_id, _flags(tag)))


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name):
    return (name.replace("void ", "").replace("aaac::", "")
            .replace("(anonymous namespace)::", "").split("(")[0])


def loop_kernel_average(rows, frag):
    """Calls-weighted average duration (ns) over every instance of a kernel family."""
    sel = [r for r in rows if frag in r["Name"]]
    calls = sum(int(r["Calls"]) for r in sel)
    total = sum(float(r["TotalDurationNs"]) for r in sel)
    return (total / calls if calls else float("nan")), calls


def kernel_stats(raw, prof, tag, out_md):
    cfg_id, desc, shapes, nl, x_bytes = workload(tag)
    N = sum(R * C for R, C in shapes)
    alg = N * 2 + N // 2 + N // 128
    rows = _rows(os.path.join(raw, "prof_%s" % tag, "run_kernel_stats.csv"))
    per = TRACE_STEPS * nl               # traced layer passes
    out = ["# Kernel durations: %s\n" % desc,
           WRITTEN_BY.format(raw=raw, prof=prof, tag=tag),
           "Command (from the repository root, on one MI355X):\n",
           "```\n%s\n```\n" % trace_cmd(raw, tag, cfg_id),
           "Source: `run_kernel_stats.csv`. Per layer a bench step runs importance on the %d "
           "activation streams, a batched init of the %d matrices, 10 x (%s; the first also sums "
           "I w^2 for the error reports), the final batched "
           "assign with its error totals, one batched pack and one batched dequant; %d steps "
           "(1 warmup + 2 timed) of %d layer%s are traced, then the decode GEMV and the AWQ "
           "pre-scale on one packed layer. Only this library's kernels are listed (input "
           "generation and copies omitted); \"per layer\" is the total divided by the %d traced "
           "layer passes.\n" % (4 if len(shapes) > 3 else 2, len(shapes),
                               "one batched fused assign + accumulate launch"
                               if WORKLOADS[tag][2] else "batched assign, batched refine",
                               TRACE_STEPS, nl, "s" if nl > 1 else "", per),
           "| kernel | calls | average (us) | min (us) | max (us) | per layer (us) |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        n = r["Name"]
        if "aaac::" not in n:
            continue
        once = ("gemv" in n) or ("awq" in n)
        per_layer = "after the steps" if once else "%.0f" % (
            float(r["TotalDurationNs"]) / 1e3 / per)
        out.append("| `%s` | %s | %.1f | %.1f | %.1f | %s |" % (
            _short(n), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, per_layer))
    out.append("")
    out.append("Per-launch algorithmic bytes of each loop launch (one layer, %s weights; the "
               "fused launch reads W and writes codes and selectors once): "
               "N x (2 + 0.5 + 1/128) B = %s B." % (format(N, ","), format(alg, ",")))
    for key, frag in loop_families(tag):
        t_ns, calls = loop_kernel_average(rows, frag)
        t = t_ns * 1e-9
        out.append("- %s (%d launches, every instance): %.1f us average -> %.0f GB/s = %.1f %% "
                   "of 8 TB/s." % (key, calls, t * 1e6, alg / t / 1e9, alg / t / PEAK * 100))
    imp = [x for x in rows if "importance_partial" in x["Name"]]
    if imp:
        t_imp = sum(float(x["TotalDurationNs"]) for x in imp) / per * 1e-9
        out.append("- importance: %.2f ms per layer for %.1f GB of activations -> %.2f TB/s." % (
            t_imp * 1e3, x_bytes / 1e9, x_bytes / t_imp / 1e12))
    gm = [x for x in rows if "gemv_kernel" in x["Name"]]
    if gm:
        gb = sum(R * C // 2 + 2 * (R * C // 128) + 2 * C + 4 * R for R, C in shapes)
        t = float(gm[0]["AverageNs"]) * 1e-9
        out.append("- decode GEMV (after the steps; batch 1, the %d packed matrices of one layer "
                   "in one launch, 512 MB read before each launch so the %.1f MB of codes, "
                   "scales, x and y come from HBM): %.1f us -> %.0f GB/s = %.1f %% of 8 TB/s."
                   % (len(shapes), gb / 1e6, t * 1e6, gb / t / 1e9, gb / t / PEAK * 100))
    aw = [x for x in rows if "awq_prescale" in x["Name"]]
    if aw:
        ab = sum(4 * R * C + 12 * C for R, C in shapes)
        tot = float(aw[0]["TotalDurationNs"]) * 1e-9 / (int(aw[0]["Calls"]) / len(shapes))
        out.append("- AWQ pre-scale (after the steps; one launch per matrix, read W and write "
                   "W diag(a): %.1f MB per layer): %.1f us per layer -> %.0f GB/s = %.1f %% of "
                   "8 TB/s." % (ab / 1e6, tot * 1e6, ab / tot / 1e9, ab / tot / PEAK * 100))
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")


def traffic(raw, prof, tag, traffic_json, out_md):
    cfg_id, desc, shapes, _, _ = workload(tag)
    N = sum(R * C for R, C in shapes)
    alg = N * 2 + N // 2 + N // 128
    with open(traffic_json) as f:
        d = json.load(f)
    out = ["# HBM traffic per launch: %s on %s\n" % (
               " and ".join(k for k, _ in loop_families(tag)), desc),
           WRITTEN_BY.format(raw=raw, prof=prof, tag=tag),
           "Two counter passes over the same command, one counter each (from the repository root, "
           "on one MI355X):\n",
           "```", pmc_cmd("FETCH_SIZE", "pmc_fetch_" + tag, raw, cfg_id, tag),
           pmc_cmd("WRITE_SIZE", "pmc_write_" + tag, raw, cfg_id, tag),
           "python -m post_weight_quantization_06_amd.pmc_traffic "
           "%s/pmc_fetch_%s/run_counter_collection.csv %s/pmc_write_%s/run_counter_collection.csv "
           "%s/hbm_traffic_assign_refine_%s.json" % (raw, tag, raw, tag, prof, tag), "```\n",
           "Calibration: bench.py copies 2^30 bytes device-to-device once before its warmup step "
           "(`__amd_rocclr_copyBuffer`, the largest copy dispatch). For that copy FETCH_SIZE reads "
           "%.1f KiB (of the 1,048,576 KiB actually read) and WRITE_SIZE %.1f KiB, so the read "
           "counter is scaled by %.4f and the write counter by %.4f.\n" % (
               d["fetch_kib_copy"], d["write_kib_copy"], d["fetch_scale"], d["write_scale"]),
           "| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read (scaled) | "
           "write (scaled) | total | algorithmic | ratio |",
           "|---|---|---|---|---|---|---|---|---|"]
    for k, v in d["kernels"].items():
        out.append("| %s | %d | %.0f | %.0f | %.1f MB | %.1f MB | %.1f MB | %.1f MB | %.3f |" % (
            k, v["dispatches"], v["fetch_kib"], v["write_kib"], v["read_bytes"] / 1e6,
            v["write_bytes"] / 1e6, v["bytes"] / 1e6, alg / 1e6, v["bytes"] / alg))
    who = ("the fused launch reads W (%.1f MB) and writes codes (%.1f MB) and selectors "
           "(%.1f MB), once per iteration" if WORKLOADS[tag][2] else
           "assign reads W (%.1f MB) and writes codes (%.1f MB) and selectors (%.1f MB); refine "
           "reads the same three") % (2 * N / 1e6, N / 2 / 1e6, N / 128 / 1e6)
    out += ["",
            "Algorithmic bytes per launch (%s weights): %s. The importance vectors and tables are "
            "not counted." % (format(N, ","), who),
            "",
            "The JSON beside this file holds the same figures with a hash of each kernel's "
            "sources; bench.py reports `roofline.traffic` only while the hash still matches."]
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")


def sq_counters(raw, prof, tag, out_md):
    cfg_id, desc, shapes, _, _ = workload(tag)
    N = sum(R * C for R, C in shapes)

    def agg(path):
        acc = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in _rows(path):
            for key, frag in loop_families(tag):
                if frag in r["Kernel_Name"]:
                    acc[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
        return acc

    a1 = agg(os.path.join(raw, "pmc_sq_" + tag, "run_counter_collection.csv"))
    a2 = agg(os.path.join(raw, "pmc_sq2_" + tag, "run_counter_collection.csv"))
    p3 = os.path.join(raw, "pmc_lds_" + tag, "run_counter_collection.csv")
    a3 = agg(p3) if os.path.exists(p3) else None
    keys = [k for k, _ in loop_families(tag)]
    out = ["# Instruction counters: %s on %s\n" % (" and ".join(keys), desc),
           WRITTEN_BY.format(raw=raw, prof=prof, tag=tag),
           "Commands (from the repository root, on one MI355X; one counter group per run):\n",
           "```", pmc_cmd(SQ1, "pmc_sq_" + tag, raw, cfg_id, tag),
           pmc_cmd(SQ2, "pmc_sq2_" + tag, raw, cfg_id, tag)]
    if a3 is not None:
        out.append(pmc_cmd(SQ3, "pmc_lds_" + tag, raw, cfg_id, tag))
    out += ["```\n",
           "Averages per dispatch (one batched launch over the %d matrices of a layer, %s "
           "weights; assign: the loop's instance without error output). SQ_INSTS_* count "
           "wave-level instructions (64 lanes), so per-weight figures are count x 64 / weights. "
           "Cycle counters are in units of 4 clocks, summed over waves.\n" % (
               len(shapes), format(N, ",")),
           "| kernel | counter | per dispatch | per weight (x64 / N) |", "|---|---|---|---|"]
    for key in keys:
        for src in (a1, a2) + ((a3,) if a3 is not None else ()):
            for c, v in src[key].items():
                mean = sum(v) / len(v)
                pw = "%.2f" % (mean * 64 / N) if c.startswith("SQ_INSTS") else ""
                out.append("| %s | %s | %.4g | %s |" % (key, c, mean, pw))

    def per_weight(src, key, c):
        v = src[key].get(c)
        return sum(v) / len(v) * 64 / N if v else float("nan")

    def share(src, key, c):
        # fraction of wave cycles: both counters are summed over waves in the same units
        v = src[key].get(c)
        w = a1[key].get("SQ_WAVE_CYCLES")
        if not v or not w:
            return float("nan")
        return 100.0 * (sum(v) / len(v)) / (sum(w) / len(w))

    def cycles(key):
        # the dispatch's active cycles (one XCD's GRBM_GUI_ACTIVE)
        g = a3[key].get("GRBM_GUI_ACTIVE")
        return (sum(g) / len(g)) / XCDS if g else float("nan")

    def busy(key, c):
        # percent of the dispatch's active cycles, per CU (the profiler's LdsUtil, VALUBusy and
        # LDSBankConflict: counter / (active cycles x CUs))
        v = a3[key].get(c)
        if not v:
            return float("nan")
        return 100.0 * (sum(v) / len(v)) / (cycles(key) * CUS)

    # the clock the kernels ran at: active cycles over the kernel trace's average duration
    trace = os.path.join(raw, "prof_%s" % tag, "run_kernel_stats.csv")
    clock = {}
    if a3 is not None and os.path.exists(trace):
        rows = _rows(trace)
        for key, frag in loop_families(tag):
            ns, calls = loop_kernel_average(rows, frag)
            if calls:
                clock[key] = cycles(key) / (ns * 1e-9)

    out += ["", "Reading (VALU issue is 64 lane-instructions per clock per CU; 256 CUs at "
                "2.4 GHz):", ""]
    if "assign" in keys:
        valu = per_weight(a1, "assign", "SQ_INSTS_VALU")
        out.append("- assign: %.1f VALU and %.1f LDS instructions per weight. VALU alone needs "
                   "%.0f us at full issue; SQ_WAIT_INST_LDS takes %.0f %% of wave time." % (
                       valu, per_weight(a1, "assign", "SQ_INSTS_LDS"),
                       N * valu / 64 / 256 / 2.4e9 * 1e6, share(a2, "assign", "SQ_WAIT_INST_LDS")))
    if "refine" in keys:
        out.append("- refine: %.1f VALU and %.2f LDS instructions (the two fp64 adds) per weight, "
                   "one workgroup of four waves per CU (128 KB of bins). Per wave: VALU busy "
                   "%.0f %%, LDS issue %.0f %%, waiting %.0f %% of its cycles." % (
                       per_weight(a1, "refine", "SQ_INSTS_VALU"),
                       per_weight(a1, "refine", "SQ_INSTS_LDS"),
                       share(a2, "refine", "SQ_ACTIVE_INST_VALU"),
                       share(a2, "refine", "SQ_ACTIVE_INST_LDS"), share(a2, "refine", "SQ_WAIT_ANY")))
    if a3 is not None:
        for key in keys:
            ghz = clock.get(key)
            out.append("- %s, per CU over the dispatch's active cycles (GRBM_GUI_ACTIVE / %d XCDs"
                       "%s): LDS busy with indexed operations %.0f %% (of which stalled on bank "
                       "conflicts %.0f %%, on address conflicts %.0f %%), VALU issuing %.0f %%." % (
                           key, XCDS,
                           "; %.2f GHz over the trace's average duration" % (ghz / 1e9)
                           if ghz else "",
                           busy(key, "SQ_LDS_IDX_ACTIVE"), busy(key, "SQ_LDS_BANK_CONFLICT"),
                           busy(key, "SQ_LDS_ADDR_CONFLICT"), busy(key, "SQ_ACTIVE_INST_VALU")))
            if ghz:
                out[-1] += (" At that clock the VALU instructions alone need %.0f us at full issue."
                            % (N * per_weight(a1, key, "SQ_INSTS_VALU") / 64 / CUS / ghz * 1e6))
    if "fused" in keys:
        valu = per_weight(a1, "fused", "SQ_INSTS_VALU")
        out.append("- fused: %.1f VALU and %.2f LDS instructions (two lookups and two fp64 adds) "
                   "per weight, one workgroup of four waves per CU (the bins). VALU alone needs "
                   "%.0f us at full issue. Per wave: VALU busy %.0f %%, LDS issue %.0f %%, "
                   "waiting %.0f %% of its cycles." % (
                       valu, per_weight(a1, "fused", "SQ_INSTS_LDS"),
                       N * valu / 64 / 256 / 2.4e9 * 1e6,
                       share(a2, "fused", "SQ_ACTIVE_INST_VALU"),
                       share(a2, "fused", "SQ_ACTIVE_INST_LDS"), share(a2, "fused", "SQ_WAIT_ANY")))
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")


def gemv_counters(raw, prof, tag, out_md):
    """Counters of the decode GEMV launches (one batched launch over the matrices of a layer)."""
    cfg_id, desc, shapes, _, _ = workload(tag)
    N = sum(R * C for R, C in shapes)
    acc = collections.defaultdict(list)
    for r in _rows(os.path.join(raw, "pmc_gemv_" + tag, "run_counter_collection.csv")):
        if GEMV in r["Kernel_Name"]:
            acc[r["Counter_Name"]].append(float(r["Counter_Value"]))
    mean = {c: sum(v) / len(v) for c, v in acc.items()}
    cmd = ("rocprofv3 --pmc %s --output-format csv -d %s/pmc_gemv_%s -o run -- python -u bench.py "
           "--config %d --steps 1 --warmup 1 --no-cpu --one-stream" % (SQG, raw, tag, cfg_id))
    out = ["# Decode GEMV counters: %s\n" % desc,
           WRITTEN_BY.format(raw=raw, prof=prof, tag=tag),
           "Command (from the repository root, on one MI355X):\n", "```", cmd, "```\n",
           "Averages over the %d GEMV launches that bench.py times after its steps (batch 1, the %d "
           "packed matrices of one layer in one launch, %s weights). SQ_INSTS_* count wave-level "
           "instructions, so per-code-byte figures are count x 64 / (weights / 2).\n"
           % (len(acc.get("SQ_INSTS_VALU", [])), len(shapes), format(N, ",")),
           "| counter | per launch | per code byte |", "|---|---|---|"]
    for c, v in mean.items():
        pb = "%.2f" % (v * 64 / (N / 2)) if c.startswith("SQ_INSTS") else ""
        out.append("| %s | %.4g | %s |" % (c, v, pb))
    cyc = mean.get("GRBM_GUI_ACTIVE", float("nan")) / XCDS

    def pct(c):
        return 100.0 * mean.get(c, float("nan")) / (cyc * CUS)

    out += ["", "Reading: per CU over the launch's active cycles (GRBM_GUI_ACTIVE / %d XCDs), the "
                "LDS is busy with indexed operations %.0f %% (stalled on bank conflicts %.0f %%) "
                "and the VALU issues %.0f %%; waves wait on LDS results %.0f %% of their cycles."
                % (XCDS, pct("SQ_LDS_IDX_ACTIVE"), pct("SQ_LDS_BANK_CONFLICT"),
                   pct("SQ_ACTIVE_INST_VALU"),
                   100.0 * mean.get("SQ_WAIT_INST_LDS", float("nan"))
                   / mean.get("SQ_WAVE_CYCLES", float("nan")))]
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")


def main(argv):
    if len(argv) not in (3, 4):
        print(__doc__)
        return 2
    raw, prof = argv[1].rstrip("/"), argv[2].rstrip("/")
    tag = argv[3] if len(argv) == 4 else "32b_model"
    kernel_stats(raw, prof, tag, os.path.join(prof, "kernel_stats_%s.md" % tag))
    tj = os.path.join(prof, "hbm_traffic_assign_refine_%s.json" % tag)
    if os.path.exists(tj):
        traffic(raw, prof, tag, tj, os.path.join(prof, "hbm_traffic_assign_refine_%s.md" % tag))
    if os.path.exists(os.path.join(raw, "pmc_sq_" + tag, "run_counter_collection.csv")):
        sq_counters(raw, prof, tag, os.path.join(prof, "sq_counters_assign_refine_%s.md" % tag))
    if os.path.exists(os.path.join(raw, "pmc_gemv_" + tag, "run_counter_collection.csv")):
        gemv_counters(raw, prof, tag, os.path.join(prof, "sq_counters_gemv_%s.md" % tag))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
