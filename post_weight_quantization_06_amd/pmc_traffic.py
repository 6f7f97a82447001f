"""HBM traffic per launch from rocprofv3 memory counters, scaled against a plain copy.

rocprofv3 reports FETCH_SIZE and WRITE_SIZE in KiB per dispatch; on this part FETCH_SIZE reads
half of the bytes a plain device copy actually reads, while WRITE_SIZE matches. Each counter is
therefore scaled by (bytes the copy moved) / (counter value of the copy), both from the same run.

Usage (after two rocprofv3 --pmc passes over the same command, one per counter):

    python -m post_weight_quantization_06_amd.pmc_traffic FETCH.csv WRITE.csv OUT.json

The summary records a hash of the kernel sources; `load_traffic` returns None once the sources
have changed, so a stale measurement is never reported against a new kernel.
"""

from __future__ import annotations

import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# kernels whose traffic is summarised: name prefixes of the dispatches (after "void "); assign is
# the loop's instance without error output, fused the one-launch iteration
KERNELS = {
    "assign": ("aaac::assign_wide_kernel<0,", "aaac::assign_kernel<0,"),
    "refine": ("aaac::refine_kernel<",),
    "fused": ("aaac::assign_refine_kernel<",),
}
KERNEL_SOURCES = {
    "assign": ["assign.hip", "assign_body.h", "lookup.h", "common.h"],
    "refine": ["refine.hip", "lookup.h", "common.h"],
    "fused": ["refine.hip", "lookup.h", "common.h"],
}


def _is(kernel_name, key):
    name = kernel_name[5:] if kernel_name.startswith("void ") else kernel_name
    return name.startswith(KERNELS[key])


COPY_BYTES = 1 << 30       # the calibration copy: 2^28 fp32 values
COPY_NAME = "copyBuffer"


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _per_kernel(path, counter):
    rows = list(csv.DictReader(open(path)))
    rows = [r for r in rows if r["Counter_Name"] == counter]
    copy = [float(r["Counter_Value"]) for r in rows if COPY_NAME in r["Kernel_Name"]]
    if not copy:
        raise SystemExit("%s: no calibration copy dispatch" % path)
    calib = max(copy)                                  # the 1 GiB copy is the largest one
    out = {}
    for key in KERNELS:
        vals = [float(r["Counter_Value"]) for r in rows if _is(r["Kernel_Name"], key)]
        if vals:
            out[key] = (sum(vals) / len(vals), len(vals))
    return calib, out


def summarize(fetch_csv, write_csv):
    fc, fk = _per_kernel(fetch_csv, "FETCH_SIZE")
    wc, wk = _per_kernel(write_csv, "WRITE_SIZE")
    f_scale = COPY_BYTES / (fc * 1024.0)
    w_scale = COPY_BYTES / (wc * 1024.0)
    res = {"copy_bytes": COPY_BYTES, "fetch_kib_copy": fc, "write_kib_copy": wc,
           "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    for key in KERNELS:
        if key in fk and key in wk:
            fb = fk[key][0] * 1024.0 * f_scale
            wb = wk[key][0] * 1024.0 * w_scale
            res["kernels"][key] = {"fetch_kib": fk[key][0], "write_kib": wk[key][0],
                                   "dispatches": fk[key][1], "read_bytes": fb,
                                   "write_bytes": wb, "bytes": fb + wb,
                                   "source_sha256": source_hash(key)}
    return res


def load_traffic(path, kernel):
    """HBM bytes per launch of `kernel` from a summary, or None if absent or stale."""
    try:
        with open(path) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    k = d.get("kernels", {}).get(kernel)
    if not k or k.get("source_sha256") != source_hash(kernel):
        return None
    return k["bytes"]


def main(argv):
    if len(argv) != 4:
        print(__doc__)
        return 2
    res = summarize(argv[1], argv[2])
    with open(argv[3], "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
