"""The benchmark's command-line contract, on the CPU: it measures one GPU
only, and it refuses to run (rather than falling back to anything) when no
GPU is visible."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, BENCH, "--gpus", str(n)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_no_gpu_no_figures():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = subprocess.run([sys.executable, BENCH, "--steps", "1", "--warmup", "0"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 1
    assert "no GPU visible" in r.stderr
    assert r.stdout == ""
