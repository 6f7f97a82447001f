"""HBM traffic from the two counter passes (no GPU): calibration against the copy, kernel
matching by name, and the source hash that retires a stale measurement."""

from __future__ import annotations

import csv
import json

from post_weight_quantization_06_amd import pmc_traffic as pt

HDR = ["Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HDR)
        for name, value in rows:
            w.writerow([name, counter, value])


def _runs(tmp_path):
    # the copy moves 2^30 bytes: FETCH_SIZE sees half of them (KiB), WRITE_SIZE all
    copy = "__amd_rocclr_copyBuffer"
    fetch = [(copy, 524288.0), (copy, 64.0),
             ("void aaac::assign_wide_kernel<0, 8, 8>(aaac::AssignBatch)", 1000.0),
             ("void aaac::assign_wide_kernel<0, 8, 8>(aaac::AssignBatch)", 1200.0),
             ("void aaac::assign_wide_kernel<1, 8, 8>(aaac::AssignBatch)", 9999.0),
             ("void aaac::refine_kernel<true, 8, false>(aaac::RefineBatch)", 2000.0),
             ("void aaac::assign_refine_kernel<8, 8, false>(aaac::RefineBatch)", 1500.0)]
    write = [(copy, 1048576.0), (copy, 128.0),
             ("void aaac::assign_wide_kernel<0, 8, 8>(aaac::AssignBatch)", 300.0),
             ("void aaac::assign_wide_kernel<0, 8, 8>(aaac::AssignBatch)", 500.0),
             ("void aaac::assign_wide_kernel<1, 8, 8>(aaac::AssignBatch)", 9999.0),
             ("void aaac::refine_kernel<true, 8, false>(aaac::RefineBatch)", 2.0),
             ("void aaac::assign_refine_kernel<8, 8, false>(aaac::RefineBatch)", 400.0)]
    f, w = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _csv(f, "FETCH_SIZE", fetch)
    _csv(w, "WRITE_SIZE", write)
    return str(f), str(w)


def test_scaled_per_kernel_bytes(tmp_path):
    f, w = _runs(tmp_path)
    res = pt.summarize(f, w)
    # the largest copy dispatch calibrates: reads x2, writes x1
    assert res["fetch_scale"] == 2.0 and res["write_scale"] == 1.0
    a = res["kernels"]["assign"]
    # only the loop's instance (<0, ...>), averaged over its dispatches
    assert a["dispatches"] == 2 and a["fetch_kib"] == 1100.0 and a["write_kib"] == 400.0
    assert a["bytes"] == 1100.0 * 1024 * 2 + 400.0 * 1024
    assert res["kernels"]["refine"]["bytes"] == 2000.0 * 1024 * 2 + 2.0 * 1024
    assert res["kernels"]["fused"]["bytes"] == 1500.0 * 1024 * 2 + 400.0 * 1024


def test_stale_summaries_are_not_reported(tmp_path):
    f, w = _runs(tmp_path)
    res = pt.summarize(f, w)
    out = tmp_path / "t.json"
    out.write_text(json.dumps(res))
    assert pt.load_traffic(str(out), "assign") == res["kernels"]["assign"]["bytes"]
    res["kernels"]["assign"]["source_sha256"] = "0" * 64
    out.write_text(json.dumps(res))
    assert pt.load_traffic(str(out), "assign") is None
    assert pt.load_traffic(str(tmp_path / "missing.json"), "refine") is None


def test_committed_summaries_match_the_current_kernels():
    """The committed HBM traffic summaries were taken on the kernel sources as they stand, so the
    bench line's roofline.traffic is reported (a kernel edit needs a new counter run)."""
    import os

    prof = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")
    for name, keys in (("hbm_traffic_assign_refine_32b_model.json", ("assign", "refine")),
                       ("hbm_traffic_assign_refine_llama8b_layer.json", ("assign", "refine")),
                       ("hbm_traffic_assign_refine_32b_model_fused.json", ("fused",))):
        for key in keys:
            assert pt.load_traffic(os.path.join(prof, name), key) is not None, (name, key)
