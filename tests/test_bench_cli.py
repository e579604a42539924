"""bench.py's command line, on the CPU: it measures one GPU and says so, and
it refuses to run without one instead of timing anything else."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=timeout, cwd=ROOT)


@pytest.mark.parametrize("n", ["2", "8", "0"])
def test_more_or_fewer_than_one_gpu_is_refused(n):
    r = run_bench("--gpus", n)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and f"--gpus {n}" in r.stderr
    assert r.stdout == ""                      # no JSON line for a run that did not happen


def test_help_names_the_options():
    r = run_bench("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--workload", "--mode", "--partition",
                "--window"):
        assert opt in r.stdout


def test_no_gpu_no_numbers():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: the bench would run")
    r = run_bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""
