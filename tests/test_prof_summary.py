"""The profile summarizer on small hand-made rocprofv3 outputs (no GPU)."""

from __future__ import annotations

import csv
import json
import os

from post_weight_quantization_06_amd import prof_summary as ps


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _fake_raw(tmp_path):
    raw = tmp_path / "raw"
    stats_hdr = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                 "StdDev"]
    _write_csv(str(raw / "prof_c2" / "run_kernel_stats.csv"), stats_hdr, [
        ["void aaac::assign_wide_kernel<false, 8, 8>(aaac::AssignBatch)", 33, 33 * 150000,
         150000, 10, 149000, 151000, 1],
        ["void aaac::refine_kernel<true, 8>(aaac::RefineBatch)", 30, 30 * 160000, 160000, 10,
         159000, 161000, 1],
        ["void aaac::importance_partial_kernel<4>(float const*, long, long, long, long, double*)",
         12, 3 * 4_000_000, 1_000_000, 10, 900000, 1100000, 1],
        ["__amd_rocclr_copyBuffer", 1, 400000, 400000, 1, 400000, 400000, 0],
    ])
    pmc_hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(str(raw / "pmc_fetch" / "run_counter_collection.csv"), pmc_hdr, [])
    sq1 = []
    for k, name in (("assign", "aaac::assign_wide_kernel<false, 8, 8>"),
                    ("refine", "void aaac::refine_kernel<true, 8>")):
        sq1 += [[name, "SQ_WAVES", 4096], [name, "SQ_INSTS_VALU", ps.N // 64 * 24],
                [name, "SQ_INSTS_LDS", ps.N // 64 * 3], [name, "SQ_WAVE_CYCLES", 1000.0]]
    _write_csv(str(raw / "pmc_sq" / "run_counter_collection.csv"), pmc_hdr, sq1)
    sq2 = []
    for name in ("aaac::assign_wide_kernel<false, 8, 8>", "void aaac::refine_kernel<true, 8>"):
        sq2 += [[name, "SQ_WAIT_INST_LDS", 30.0], [name, "SQ_ACTIVE_INST_VALU", 440.0],
                [name, "SQ_ACTIVE_INST_LDS", 300.0], [name, "SQ_WAIT_ANY", 140.0]]
    _write_csv(str(raw / "pmc_sq2" / "run_counter_collection.csv"), pmc_hdr, sq2)
    prof = tmp_path / "prof"
    prof.mkdir()
    kern = {"dispatches": 22, "fetch_kib": 1.0, "write_kib": 1.0, "read_bytes": 2.0 * ps.N,
            "write_bytes": float(ps.N // 2 + ps.N // 128), "bytes": float(ps.ALG)}
    (prof / "hbm_traffic_assign_refine_llama8b_layer.json").write_text(json.dumps({
        "fetch_kib_copy": 524288.0, "write_kib_copy": 1048576.0, "fetch_scale": 2.0,
        "write_scale": 1.0, "kernels": {"assign": kern, "refine": dict(kern)}}))
    return raw, prof


def test_summaries_from_fake_runs(tmp_path):
    raw, prof = _fake_raw(tmp_path)
    assert ps.main(["prof_summary", str(raw), str(prof) + "/"]) == 0
    stats = (prof / "kernel_stats_llama8b_layer.md").read_text()
    # 546,963,456 B in 150 us and 160 us
    assert "- assign: 150.0 us average -> 3646 GB/s = 45.6 % of 8 TB/s." in stats
    assert "- refine: 160.0 us average -> 3419 GB/s = 42.7 % of 8 TB/s." in stats
    assert "copyBuffer" not in stats
    assert "-d %s/prof_c2" % raw in stats
    traffic = (prof / "hbm_traffic_assign_refine_llama8b_layer.md").read_text()
    assert "| assign | 22 |" in traffic and "| 1.000 |" in traffic
    assert "assign reads 1.000x the bf16 weights and writes 1.000x" in traffic
    sq = (prof / "sq_counters_assign_refine_llama8b_layer.md").read_text()
    # 24 VALU per weight; the cycle shares are ratios of the fake counters
    assert "- assign: 24.0 VALU and 3.0 LDS instructions per weight." in sq
    assert "VALU busy 44 %, LDS issue 30 %, waiting 14 %" in sq
