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


def test_tile_skip_switch_accepted():
    """--no-tile-skip (the A/B of the tile classes) is a known option: without
    a GPU the run stops at the GPU check, not at the argument parser."""
    import torch
    if torch.cuda.is_available():
        import pytest
        pytest.skip("a GPU is present")
    r = _run("--no-tile-skip", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2 and "needs a GPU" in r.stderr and "unrecognized" not in r.stderr


def test_attention_flop_hand_count():
    """The metric's FLOP count against a count done by hand. One head, 2 query
    rows, 3 keys, head dim 4: Q.K^T is 2 x 3 dot products of length 4, each 4
    multiplies and 4 adds = 8 FLOP, 48 in all; P.V is 2 rows x 4 dims, each a
    sum over 3 keys of 3 multiplies and 3 adds = 6 FLOP, 48 in all; total 96.
    Batches and heads multiply it: B = 2, H = 3 gives 576."""
    sys.path.insert(0, ROOT)
    import bench
    assert bench.attention_flop(1, 1, 2, 3, 4) == 96.0
    assert bench.attention_flop(2, 3, 2, 3, 4) == 576.0
    # the headline: 4 * 56 * 107,126^2 * 128
    assert bench.attention_flop(1, 56, 107126, 107126, 128) == 329039295004672.0
