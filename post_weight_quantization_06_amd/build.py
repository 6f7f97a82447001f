"""Build the HIP library libaaac.so in-tree for gfx950.

Usage: python -m post_weight_quantization_06_amd.build   (or build() from Python)
Every call compiles again from source: each .hip file to an object (in parallel), then one link.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libaaac.so")
SOURCES = ["abi.hip", "assign.hip", "refine.hip", "importance.hip", "init.hip", "pack.hip",
           "awq.hip", "gemv.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout or "") + (res.stderr or "")
    # the host pass does not know the gfx-only feature flag; that warning is expected
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    return res.returncode, lines


def build(verbose=False, extra_flags=(), jobs=None):
    tmpdir = tempfile.mkdtemp(prefix="aaac_build_")
    try:
        objs, cmds = [], []
        for s in SOURCES:
            obj = os.path.join(tmpdir, s.replace(".hip", ".o"))
            objs.append(obj)
            cmds.append([hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c",
                         os.path.join(CSRC, s), "-o", obj])
        jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for cmd, (rc, lines) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError("hipcc failed (%d):\n%s" % (rc, "\n".join(lines)))
            if verbose and lines:
                print("\n".join(lines))
        tmp = LIB + ".tmp"
        link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, lines = _run(link)
        if rc != 0:
            raise RuntimeError("hipcc link failed (%d):\n%s" % (rc, "\n".join(lines)))
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
