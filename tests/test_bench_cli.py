"""Command-line contract of bench.py that holds without a GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    # One stage on one GPU is what the benchmark measures; N > 1 exits non-zero
    # before touching any device, with a message saying so.
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""
