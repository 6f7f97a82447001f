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


def test_algorithmic_bytes_per_launch():
    """Read W (2 B), write or read the codes (0.5 B) and the selectors (1/S B) per weight: the
    32B-shaped layer's figure quoted with the roofline, and the 8B-shaped layer's with S = 16."""
    sys.path.insert(0, ROOT)
    import bench
    from synth import layers as syn

    n32 = sum(m.rows * m.cols for m in syn.config(5).matrices)
    assert n32 == 487587840
    assert bench.algorithmic_bytes(n32, 128) == 1222778880
    n8 = sum(m.rows * m.cols for m in syn.config(2).matrices)
    assert bench.algorithmic_bytes(n8, 128) == 546963456
    assert bench.algorithmic_bytes(n8, 16) == n8 * 2 + n8 // 2 + n8 // 16
