"""Text summaries of rocprofv3 runs of bench.py on the 8B-shaped decoder layer.

Turns the raw rocprofv3 output of the runs below (one counter group per run, all writing under
one folder RAW) into the short Markdown summaries kept beside the traffic JSON:

    rocprofv3 --kernel-trace --stats --output-format csv -d RAW/prof_c2 -o run -- \\
        python -u bench.py --steps 2 --warmup 1 --no-cpu --one-stream
    rocprofv3 --pmc FETCH_SIZE ... -d RAW/pmc_fetch ...      (the same bench command, 1 step)
    rocprofv3 --pmc WRITE_SIZE ... -d RAW/pmc_write ...
    rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU ... -d RAW/pmc_sq ...
    rocprofv3 --pmc SQ_WAIT_ANY SQ_WAIT_INST_LDS ... -d RAW/pmc_sq2 ...
    python -m post_weight_quantization_06_amd.pmc_traffic FETCH.csv WRITE.csv TRAFFIC.json

Usage (from the repository root):

    python -m post_weight_quantization_06_amd.prof_summary RAW PROFILES

PROFILES holds hbm_traffic_assign_refine_llama8b_layer.json and receives the three .md files,
whose command lines name RAW and PROFILES as given.
"""

from __future__ import annotations

import collections
import csv
import json
import os
import sys

# the 8B-shaped layer: [out, in] of q, k, v, o, gate, up, down
MATS = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096), (14336, 4096),
        (4096, 14336)]
N = sum(r * c for r, c in MATS)                      # 218,103,808 weights
ALG = N * 2 + N // 2 + N // 128                      # bytes per assign or refine launch
X_BYTES = 4 * 262144 * (3 * 4096 + 14336)            # the four activation streams, fp32
PEAK = 8e12

TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d {raw}/prof_c2 -o run "
             "-- python -u bench.py --steps 2 --warmup 1 --no-cpu --one-stream")
SQ1 = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU SQ_WAVE_CYCLES SQ_BUSY_CYCLES "
       "SQ_WAIT_INST_ANY SQ_INSTS_VMEM_RD")
SQ2 = ("SQ_WAIT_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT "
       "SQ_ACTIVE_INST_ANY")
WRITTEN_BY = ("Summary written by `python -m post_weight_quantization_06_amd.prof_summary {raw} "
              "{prof}` from the raw output of the commands below.\n")


def _pmc_cmd(counters, out, raw):
    return ("rocprofv3 --pmc %s --output-format csv -d %s/%s -o run -- python -u bench.py "
            "--steps 1 --warmup 1 --no-cpu --one-stream" % (counters, raw, out))


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def kernel_stats(raw, prof, out_md):
    rows = _rows(os.path.join(raw, "prof_c2", "run_kernel_stats.csv"))
    out = ["# Kernel durations: 8B-shaped decoder layer (218,103,808 weights, g=128, S=128, n=16, "
           "10 iterations)\n",
           WRITTEN_BY.format(raw=raw, prof=prof),
           "Command (from the repository root, on one MI355X):\n",
           "```\n%s\n```\n" % TRACE_CMD.format(raw=raw),
           "Source: `run_kernel_stats.csv`. One bench step runs importance on the 4 activation "
           "streams, a batched init of the 7 matrices, 10 x (batched assign, batched refine), a final batched "
           "assign, then one batched pack and one batched dequant; 3 steps (1 warmup + 2 timed) are traced, then "
           "the decode GEMV (9 launches) and the AWQ pre-scale (3 rounds of 7 launches) on the "
           "packed layer. Only this library's kernels are listed (input generation and copies "
           "omitted); \"per step\" is the total divided by 3.\n",
           "| kernel | calls | average (us) | min (us) | max (us) | per step (us) |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        n = r["Name"]
        if "aaac::" not in n:
            continue
        short = (n.replace("void ", "").replace("aaac::", "")
                 .replace("(anonymous namespace)::", "").split("(")[0])
        once = ("gemv" in n) or ("awq" in n)
        per_step = "after the steps" if once else "%.0f" % (float(r["TotalDurationNs"]) / 1e3 / 3)
        out.append("| `%s` | %s | %.1f | %.1f | %.1f | %s |" % (
            short, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, per_step))
    out.append("")
    out.append("Per-launch algorithmic bytes of assign and of refine: 218,103,808 x (2 + 0.5 + "
               "1/128) B = %s B." % format(ALG, ","))
    for key, frag in (("assign", "assign_wide_kernel"), ("refine", "refine_kernel<")):
        r = [x for x in rows if frag in x["Name"]][0]
        t = float(r["AverageNs"]) * 1e-9
        out.append("- %s: %.1f us average -> %.0f GB/s = %.1f %% of 8 TB/s." % (
            key, t * 1e6, ALG / t / 1e9, ALG / t / PEAK * 100))
    imp = [x for x in rows if "importance_partial" in x["Name"]][0]
    t_imp = float(imp["TotalDurationNs"]) / 3 * 1e-9
    out.append("- importance: %.2f ms per step for %.1f GB of activations -> %.2f TB/s." % (
        t_imp * 1e3, X_BYTES / 1e9, X_BYTES / t_imp / 1e12))
    gm = [x for x in rows if "gemv_kernel" in x["Name"]]
    if gm:
        gb = sum(R * C // 2 + 2 * (R * C // 128) + 2 * C + 4 * R for R, C in MATS)
        t = float(gm[0]["AverageNs"]) * 1e-9
        fetch = [float(x["Counter_Value"])
                 for x in _rows(os.path.join(raw, "pmc_fetch", "run_counter_collection.csv"))
                 if "gemv_kernel" in x["Kernel_Name"]]
        fb = sum(fetch) / len(fetch) * 1024 * 2 if fetch else float("nan")
        out.append("- decode GEMV (after the steps; batch 1, all 7 packed matrices in one launch, "
                   "512 MB read before each launch so the %.1f MB of codes, scales, x and y come "
                   "from HBM): %.1f us -> %.0f GB/s = %.1f %% of 8 TB/s; FETCH_SIZE x 2 = %.1f MB "
                   "per launch (no re-reads)." % (gb / 1e6, t * 1e6, gb / t / 1e9,
                                                 gb / t / PEAK * 100, fb / 1e6))
    aw = [x for x in rows if "awq_prescale" in x["Name"]]
    if aw:
        ab = sum(4 * R * C + 12 * C for R, C in MATS)
        tot = float(aw[0]["TotalDurationNs"]) * 1e-9 / (int(aw[0]["Calls"]) / 7)
        out.append("- AWQ pre-scale (after the steps; one launch per matrix, read W and write "
                   "W diag(a): %.1f MB per layer): %.1f us per layer -> %.0f GB/s = %.1f %% of "
                   "8 TB/s." % (ab / 1e6, tot * 1e6, ab / tot / 1e9, ab / tot / PEAK * 100))
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")


def traffic(raw, prof, traffic_json, out_md):
    with open(traffic_json) as f:
        d = json.load(f)
    out = ["# HBM traffic per launch: assign and refine on the 8B-shaped decoder layer\n",
           WRITTEN_BY.format(raw=raw, prof=prof),
           "Two counter passes over the same command, one counter each (from the repository root, "
           "on one MI355X):\n",
           "```", _pmc_cmd("FETCH_SIZE", "pmc_fetch", raw), _pmc_cmd("WRITE_SIZE", "pmc_write", raw),
           "python -m post_weight_quantization_06_amd.pmc_traffic "
           "%s/pmc_fetch/run_counter_collection.csv %s/pmc_write/run_counter_collection.csv "
           "%s/hbm_traffic_assign_refine_llama8b_layer.json" % (raw, raw, prof), "```\n",
           "Calibration: bench.py copies 2^30 bytes device-to-device once before its warmup step "
           "(`__amd_rocclr_copyBuffer`, the largest copy dispatch). For that copy FETCH_SIZE reads "
           "%.1f KiB (half of the 1,048,576 KiB actually read) and WRITE_SIZE %.1f KiB, so the read "
           "counter is scaled by %.4f and the write counter by %.4f.\n" % (
               d["fetch_kib_copy"], d["write_kib_copy"], d["fetch_scale"], d["write_scale"]),
           "| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read (scaled) | "
           "write (scaled) | total | algorithmic | ratio |",
           "|---|---|---|---|---|---|---|---|---|"]
    for k, v in d["kernels"].items():
        out.append("| %s | %d | %.0f | %.0f | %.1f MB | %.1f MB | %.1f MB | %.1f MB | %.3f |" % (
            k, v["dispatches"], v["fetch_kib"], v["write_kib"], v["read_bytes"] / 1e6,
            v["write_bytes"] / 1e6, v["bytes"] / 1e6, ALG / 1e6, v["bytes"] / ALG))
    a = d["kernels"]["assign"]
    r = d["kernels"]["refine"]
    w_bytes = 2 * N
    cs_bytes = N // 2 + N // 128
    out += ["",
            "Algorithmic bytes per launch (218,103,808 weights): assign reads W (%.1f MB) and "
            "writes codes (%.1f MB) and selectors (%.1f MB); refine reads the same three. The "
            "importance vectors and tables (under 0.2 MB) are not counted." % (
                w_bytes / 1e6, N / 2 / 1e6, N / 128 / 1e6),
            "",
            "- assign reads %.3fx the bf16 weights and writes %.3fx its codes + selectors. The "
            "selector bytes (one per 128 weights) are written as single bytes from different "
            "waves; partially written lines are the likely source of the extra write traffic." % (
                a["read_bytes"] / w_bytes, a["write_bytes"] / cs_bytes),
            "- refine reads %.3fx W + codes + selectors." % (r["read_bytes"] / ALG),
            "- Neither kernel re-reads its inputs: both are limited by instruction issue, not by "
            "HBM bytes.",
            "",
            "The JSON beside this file holds the same figures with a hash of each kernel's "
            "sources; bench.py reports `roofline.traffic` only while the hash still matches."]
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")


def sq_counters(raw, prof, out_md):
    def agg(path):
        acc = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in _rows(path):
            for key, frag in (("assign", "assign_wide_kernel"), ("refine", "aaac::refine_kernel<")):
                if frag in r["Kernel_Name"]:
                    acc[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
        return acc

    a1 = agg(os.path.join(raw, "pmc_sq", "run_counter_collection.csv"))
    a2 = agg(os.path.join(raw, "pmc_sq2", "run_counter_collection.csv"))
    out = ["# Instruction counters: assign and refine on the 8B-shaped decoder layer\n",
           WRITTEN_BY.format(raw=raw, prof=prof),
           "Commands (from the repository root, on one MI355X; one counter group per run):\n",
           "```", _pmc_cmd(SQ1, "pmc_sq", raw), _pmc_cmd(SQ2, "pmc_sq2", raw), "```\n",
           "Averages per dispatch (one batched launch over all 7 matrices, 218,103,808 weights). "
           "SQ_INSTS_* count wave-level instructions (64 lanes), so per-weight figures are count x "
           "64 / weights. Cycle counters are in units of 4 clocks, summed over waves.\n",
           "| kernel | counter | per dispatch | per weight (x64 / N) |", "|---|---|---|---|"]
    for key in ("assign", "refine"):
        for src in (a1, a2):
            for c, v in src[key].items():
                mean = sum(v) / len(v)
                pw = "%.2f" % (mean * 64 / N) if c.startswith("SQ_INSTS") else ""
                out.append("| %s | %s | %.4g | %s |" % (key, c, mean, pw))

    def per_weight(src, key, c):
        v = src[key][c]
        return sum(v) / len(v) * 64 / N

    def share(src, key, c):
        # fraction of wave cycles: both counters are summed over waves in the same units
        v = src[key][c]
        w = a1[key]["SQ_WAVE_CYCLES"]
        return 100.0 * (sum(v) / len(v)) / (sum(w) / len(w))

    valu = per_weight(a1, "assign", "SQ_INSTS_VALU")
    out += ["", "Reading (VALU issue is 64 lane-instructions per clock per CU; 256 CUs at "
                "2.4 GHz):", "",
            "- assign: %.1f VALU and %.1f LDS instructions per weight. VALU alone needs %.0f us "
            "at full issue; SQ_WAIT_INST_LDS (waiting to issue LDS instructions, bank conflicts of "
            "the random record reads) takes %.0f %% of wave time." % (
                valu, per_weight(a1, "assign", "SQ_INSTS_LDS"), N * valu / 64 / 256 / 2.4e9 * 1e6,
                share(a2, "assign", "SQ_WAIT_INST_LDS")),
            "- refine: %.1f VALU and %.2f LDS instructions (the two fp64 adds) per weight, one "
            "workgroup of four waves per CU (128 KB of bins). Per wave: VALU busy %.0f %%, LDS "
            "issue %.0f %%, waiting %.0f %% of its cycles; one wave per SIMD cannot overlap "
            "them." % (
                per_weight(a1, "refine", "SQ_INSTS_VALU"), per_weight(a1, "refine", "SQ_INSTS_LDS"),
                share(a2, "refine", "SQ_ACTIVE_INST_VALU"), share(a2, "refine", "SQ_ACTIVE_INST_LDS"),
                share(a2, "refine", "SQ_WAIT_ANY"))]
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")


def main(argv):
    if len(argv) != 3:
        print(__doc__)
        return 2
    raw, prof = argv[1].rstrip("/"), argv[2].rstrip("/")
    kernel_stats(raw, prof, os.path.join(prof, "kernel_stats_llama8b_layer.md"))
    traffic(raw, prof, os.path.join(prof, "hbm_traffic_assign_refine_llama8b_layer.json"),
            os.path.join(prof, "hbm_traffic_assign_refine_llama8b_layer.md"))
    sq_counters(raw, prof, os.path.join(prof, "sq_counters_assign_refine_llama8b_layer.md"))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
