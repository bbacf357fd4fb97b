"""bench.py's host-side contract (no GPU needed): more than one GPU is
refused with a message, and without a GPU it fails loudly instead of
falling back to anything."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("launches", ["fused", "clipped"])
def test_one_call_steps_and_8bit_together_are_refused_or_need_a_gpu(launches):
    r = run("--launches", launches, "--state8")
    assert r.returncode != 0 and r.stdout.strip() == ""


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_no_gpu_fails_loudly():
    r = run("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr
    assert r.stdout.strip() == ""
