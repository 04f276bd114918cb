"""bench.py's contract on a host without a GPU: more than one GPU is refused
with a message (this build runs on one GPU), and without a visible GPU the
bench fails loudly instead of falling back to anything."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line


def test_no_gpu_fails_loudly():
    import pytest
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: the real bench runs instead")
    r = run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert "no GPU" in r.stderr
    assert r.stdout.strip() == ""
