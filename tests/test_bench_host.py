"""bench.py's host-side contract (no GPU): it measures one GPU and says so for any other count."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    for n in ("2", "8"):
        res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n,
                              "--no-cpu"], capture_output=True, text=True, timeout=120)
        assert res.returncode == 2
        assert "one GPU only" in res.stderr and ("--gpus %s" % n) in res.stderr
        assert res.stdout == ""
