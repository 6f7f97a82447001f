"""The profile summarizer on small hand-made rocprofv3 outputs (no GPU)."""

from __future__ import annotations

import csv
import json
import os

from post_weight_quantization_06_amd import prof_summary as ps

TAG = "llama8b_layer"
N = 218103808                                  # weights of the 8B-shaped layer
ALG = N * 2 + N // 2 + N // 128


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
    _write_csv(str(raw / ("prof_" + TAG) / "run_kernel_stats.csv"), stats_hdr, [
        ["void aaac::assign_wide_kernel<0, 8, 8>(aaac::AssignBatch)", 30, 30 * 150000,
         150000, 10, 149000, 151000, 1],
        ["void aaac::assign_wide_kernel<1, 8, 8>(aaac::AssignBatch)", 3, 3 * 180000,
         180000, 1, 179000, 181000, 1],
        # two refine instances: 27 plain launches at 150 us, 3 that also sum I w^2 at 240 us
        ["void aaac::refine_kernel<true, 8, false>(aaac::RefineBatch)", 27, 27 * 150000, 150000,
         10, 149000, 151000, 1],
        ["void aaac::refine_kernel<true, 8, true>(aaac::RefineBatch)", 3, 3 * 240000, 240000,
         1, 239000, 241000, 1],
        ["void aaac::importance_partial_kernel<4>(float const*, long, long, long, long, double*)",
         12, 3 * 4_000_000, 1_000_000, 10, 900000, 1100000, 1],
        ["__amd_rocclr_copyBuffer", 1, 400000, 400000, 1, 400000, 400000, 0],
    ])
    pmc_hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    sq1, sq2 = [], []
    for name in ("aaac::assign_wide_kernel<0, 8, 8>", "void aaac::refine_kernel<true, 8, false>"):
        sq1 += [[name, "SQ_WAVES", 4096], [name, "SQ_INSTS_VALU", N // 64 * 24],
                [name, "SQ_INSTS_LDS", N // 64 * 3], [name, "SQ_WAVE_CYCLES", 1000.0]]
        sq2 += [[name, "SQ_WAIT_INST_LDS", 30.0], [name, "SQ_ACTIVE_INST_VALU", 440.0],
                [name, "SQ_ACTIVE_INST_LDS", 300.0], [name, "SQ_WAIT_ANY", 140.0]]
    _write_csv(str(raw / ("pmc_sq_" + TAG) / "run_counter_collection.csv"), pmc_hdr, sq1)
    _write_csv(str(raw / ("pmc_sq2_" + TAG) / "run_counter_collection.csv"), pmc_hdr, sq2)
    prof = tmp_path / "prof"
    prof.mkdir()
    kern = {"dispatches": 22, "fetch_kib": 1.0, "write_kib": 1.0, "read_bytes": 2.0 * N,
            "write_bytes": float(N // 2 + N // 128), "bytes": float(ALG)}
    (prof / ("hbm_traffic_assign_refine_%s.json" % TAG)).write_text(json.dumps({
        "fetch_kib_copy": 524288.0, "write_kib_copy": 1048576.0, "fetch_scale": 2.0,
        "write_scale": 1.0, "kernels": {"assign": kern, "refine": dict(kern)}}))
    return raw, prof


def test_summaries_from_fake_runs(tmp_path):
    raw, prof = _fake_raw(tmp_path)
    assert ps.main(["prof_summary", str(raw), str(prof) + "/", TAG]) == 0
    stats = (prof / ("kernel_stats_%s.md" % TAG)).read_text()
    # 546,963,456 B in 150 us; refine averages its two instances: (27 x 150 + 3 x 240) / 30 = 159
    assert "- assign (30 launches, every instance): 150.0 us average -> 3646 GB/s = 45.6 %" in stats
    assert "- refine (30 launches, every instance): 159.0 us average -> 3440 GB/s = 43.0 %" in stats
    assert "copyBuffer" not in stats
    assert "-d %s/prof_%s" % (raw, TAG) in stats
    traffic = (prof / ("hbm_traffic_assign_refine_%s.md" % TAG)).read_text()
    assert "| assign | 22 |" in traffic and "| 1.000 |" in traffic
    sq = (prof / ("sq_counters_assign_refine_%s.md" % TAG)).read_text()
    # 24 VALU per weight; the cycle shares are ratios of the fake counters
    assert "- assign: 24.0 VALU and 3.0 LDS instructions per weight." in sq
    assert "VALU busy 44 %, LDS issue 30 %, waiting 14 %" in sq


def test_unit_busy_lines_from_the_lds_pass(tmp_path):
    raw, prof = _fake_raw(tmp_path)
    pmc_hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    cycles = 700000.0                    # the dispatch's active GPU cycles
    lds = []
    for name, idx, valu in (("aaac::assign_wide_kernel<0, 8, 8>", 0.25, 0.86),
                            ("void aaac::refine_kernel<true, 8, false>", 0.93, 0.40)):
        lds += [[name, "SQ_LDS_IDX_ACTIVE", idx * cycles * 256],
                [name, "SQ_LDS_BANK_CONFLICT", 0.10 * cycles * 256],
                [name, "SQ_LDS_ADDR_CONFLICT", 0.0],
                [name, "SQ_ACTIVE_INST_VALU", valu * cycles * 256],
                [name, "GRBM_GUI_ACTIVE", cycles * ps.XCDS]]
    _write_csv(str(raw / ("pmc_lds_" + TAG) / "run_counter_collection.csv"), pmc_hdr, lds)
    assert ps.main(["prof_summary", str(raw), str(prof), TAG]) == 0
    sq = (prof / ("sq_counters_assign_refine_%s.md" % TAG)).read_text()
    assert "GRBM_GUI_ACTIVE -d %s/pmc_lds_%s" % (raw, TAG) in sq.replace("--output-format csv ", "")
    # 700,000 cycles in the 150 us average of the fake trace: 4.67 GHz
    assert ("- assign, per CU over the dispatch's active cycles (GRBM_GUI_ACTIVE / 8 XCDs; 4.67 "
            "GHz over the trace's average duration): LDS busy with indexed operations 25 % (of "
            "which stalled on bank conflicts 10 %, on address conflicts 0 %), VALU issuing "
            "86 %.") in sq
    assert "LDS busy with indexed operations 93 %" in sq


def test_gemv_counter_summary(tmp_path):
    raw, prof = _fake_raw(tmp_path)
    pmc_hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    cycles = 180000.0
    name = "void aaac::(anonymous namespace)::gemv_kernel<1, 1, 1, true>(aaac::GemvBatch)"
    rows = [[name, "SQ_INSTS_VALU", N // 2 // 64 * 3.0], [name, "SQ_INSTS_LDS", N // 2 // 64],
            [name, "SQ_LDS_IDX_ACTIVE", 0.66 * cycles * 256],
            [name, "SQ_LDS_BANK_CONFLICT", 0.38 * cycles * 256],
            [name, "SQ_ACTIVE_INST_VALU", 0.44 * cycles * 256],
            [name, "SQ_WAIT_INST_LDS", 17.0], [name, "SQ_WAVE_CYCLES", 100.0],
            [name, "GRBM_GUI_ACTIVE", cycles * ps.XCDS],
            ["void aaac::refine_kernel<true, 8, false>(aaac::RefineBatch)", "SQ_INSTS_VALU", 1.0]]
    _write_csv(str(raw / ("pmc_gemv_" + TAG) / "run_counter_collection.csv"), pmc_hdr, rows)
    assert ps.main(["prof_summary", str(raw), str(prof), TAG]) == 0
    g = (prof / ("sq_counters_gemv_%s.md" % TAG)).read_text()
    assert "| SQ_INSTS_VALU | " in g and "| 3.00 |" in g and "| 1.00 |" in g
    assert ("the LDS is busy with indexed operations 66 % (stalled on bank conflicts 38 %) and the "
            "VALU issues 44 %; waves wait on LDS results 17 % of their cycles.") in g


def test_workloads_match_the_registry():
    cfg_id, _, shapes, layers, x_bytes = ps.workload("32b_model")
    assert cfg_id == 5 and layers == 64 and len(shapes) == 7
    assert sum(R * C for R, C in shapes) == 487587840
    assert x_bytes == 4 * 524288 * (3 * 5120 + 27648)


def test_fused_workload_summaries(tmp_path):
    tag = "32b_model_fused"
    n32 = 487587840
    alg32 = n32 * 2 + n32 // 2 + n32 // 128
    raw = tmp_path / "raw"
    stats_hdr = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                 "StdDev"]
    _write_csv(str(raw / ("prof_" + tag) / "run_kernel_stats.csv"), stats_hdr, [
        ["void aaac::assign_refine_kernel<8, 8, false>(aaac::RefineBatch)", 1728, 1728 * 800000,
         800000, 50, 790000, 810000, 1],
        ["void aaac::assign_refine_kernel<8, 8, true>(aaac::RefineBatch)", 192, 192 * 800000,
         800000, 5, 790000, 810000, 1],
        ["void aaac::assign_wide_kernel<1, 8, 8>(aaac::AssignBatch)", 192, 192 * 400000,
         400000, 5, 399000, 401000, 1],
    ])
    pmc_hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    name = "void aaac::assign_refine_kernel<8, 8, false>"
    _write_csv(str(raw / ("pmc_sq_" + tag) / "run_counter_collection.csv"), pmc_hdr,
               [[name, "SQ_INSTS_VALU", n32 // 64 * 34], [name, "SQ_INSTS_LDS", n32 // 64 * 4],
                [name, "SQ_WAVE_CYCLES", 1000.0]])
    _write_csv(str(raw / ("pmc_sq2_" + tag) / "run_counter_collection.csv"), pmc_hdr,
               [[name, "SQ_ACTIVE_INST_VALU", 560.0], [name, "SQ_ACTIVE_INST_LDS", 130.0],
                [name, "SQ_WAIT_ANY", 250.0]])
    prof = tmp_path / "prof"
    prof.mkdir()
    assert ps.main(["prof_summary", str(raw), str(prof), tag]) == 0
    stats = (prof / ("kernel_stats_%s.md" % tag)).read_text()
    # every instance of the fused kernel, no assign or refine lines
    assert "- fused (1920 launches, every instance): 800.0 us average -> %.0f GB/s" % (
        alg32 / 800e-6 / 1e9) in stats
    assert "- assign (" not in stats and "- refine (" not in stats
    assert "--config 5 --fused --steps 2" in stats
    sq = (prof / ("sq_counters_assign_refine_%s.md" % tag)).read_text()
    assert "- fused: 34.0 VALU and 4.00 LDS" in sq
    assert "VALU busy 56 %, LDS issue 13 %, waiting 25 %" in sq
    assert not (prof / ("hbm_traffic_assign_refine_%s.md" % tag)).exists()
