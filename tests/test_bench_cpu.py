"""bench.py contract checks that need no GPU: it measures one GPU only and
says so when asked for more."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "one GPU" in r.stdout


def test_help_lists_the_legs():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--gpus", "--no-cpu-baseline", "--no-backward", "--no-convergence"):
        assert flag in r.stdout
