"""bench.py's contract checks that need no GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert run.returncode == 2
    assert "one GPU" in run.stderr + run.stdout
    assert run.stdout.strip() == ""          # no JSON line
