"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with a message (this is a single-GPU kernel), and so is a host
without a GPU; neither run times anything."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, env=env)


def test_refuses_more_than_one_gpu():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_refuses_distributed_launch():
    env = dict(os.environ, WORLD_SIZE="4")
    r = _run(env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_needs_a_gpu_here():
    import torch
    if torch.cuda.is_available():
        import pytest
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 2 and "needs a GPU" in r.stderr
