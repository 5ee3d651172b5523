"""bench.py refuses what it does not measure before touching a GPU (CPU tests)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "single" in r.stderr


def test_fused_step_needs_the_plain_path_without_shared_blocks():
    for args in (("--step", "fused", "--workload", "fp8_prefix"),
                 ("--step", "fused", "--decode-path", "multi")):
        r = _run(*args)
        assert r.returncode == 1 and "--step fused needs" in r.stderr
