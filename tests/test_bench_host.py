"""bench.py's command line on the host: more than one GPU is refused with a
message (the benchmark measures one GPU), and without a GPU it exits with an
error instead of measuring anything on the CPU."""

import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = _bench("--gpus", n, "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert not r.stdout.strip()


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the path taken without a GPU")
def test_no_gpu_is_an_error():
    r = _bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "needs a ROCm GPU" in r.stderr
    assert not r.stdout.strip()
