"""Command-line contract of bench.py that holds without a GPU: more than one
GPU is refused with a message, and without a GPU the script exits non-zero
instead of falling back to the CPU."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the behaviour without a GPU")
def test_no_gpu_exits_nonzero_without_a_bench_line():
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert not any(line.startswith("{") for line in r.stdout.splitlines())
