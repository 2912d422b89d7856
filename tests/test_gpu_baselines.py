"""GPU parity of the two comparison baselines against the fp64 oracle, through
the C ABI, at the usual gates (max|dO| <= 1e-2, max|dLSE| <= 1e-3, relative
1e-2):

- dense-bias: the bias of every (query, key) pair written to HBM as a dense
  fp32 tensor, then read by the attention pass (the dense bias tensor the
  "Three backends" section says the Flash Partitions evaluation avoids);
- frame-loop: the fused pass launched once per query range (one per target
  latent frame and one per run of other rows), the per-frame attention loop
  that the one-pass kernels of that section drop.

Both compute the same O and LSE as the fused mode.
"""
import numpy as np
import pytest
import torch

import tara_inputs as ti
from tara_testlib import compare, log, qkv_random, run_gpu, run_oracle, sample_rows

pytestmark = pytest.mark.gpu

DEF = ti.Params()
BIND = ti.Params(window=0.10, falloff=0.40, strength=3.0, cap=8.0, binding=True, gains=(1.25, 0.75, 0.75))
CHAIN = ti.Params(window=0.10, falloff=0.40, strength=3.0, cap=8.0, binding=True, gains=(1.25, 0.75, 0.75),
                  chained=((0.8, 1.4, 1.1),))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def small_layout(mask=False, pictures=3, planes=1):
    return ti.make_layout(6, (6, 10), (6, 10), pictures, 40, 37, mask=mask, mask_planes=planes)


def check(q, k, v, lay, p, what, **kw):
    o, l = run_gpu(q, k, v, lay, p, **kw)
    ro, rl = run_oracle(q, k, v, lay, p, use_mask=kw.get("use_mask", True))
    return compare(o.numpy(), l.numpy(), ro, rl, what=what)


def frame_loop(lay):
    b = ti.frame_loop_bounds(lay)
    return dict(mode="frame-loop", partitions=len(b) - 1, bounds=b)


@pytest.mark.parametrize("d", [128, 64])
def test_dense_bias_small(d):
    lay = small_layout(mask=True)
    q, k, v = qkv_random(1, 2, lay.n, d, seed=120 + d)
    check(q, k, v, lay, DEF, f"dense-bias defaults d={d}", mode="dense-bias")
    check(q, k, v, lay, BIND, f"dense-bias binding d={d}", mode="dense-bias")


def test_dense_bias_chained_shuffled_batched():
    lay = small_layout(mask=True, planes=2)
    q, k, v = qkv_random(2, 2, lay.n, 128, seed=123)
    check(q, k, v, lay, CHAIN, "dense-bias chained B=2", mode="dense-bias")
    sh = lay.permuted(np.random.default_rng(124).permutation(lay.n))
    q, k, v = qkv_random(1, 2, lay.n, 128, seed=125)
    check(q, k, v, sh, BIND, "dense-bias shuffled", mode="dense-bias")


@pytest.mark.parametrize("d", [128, 64])
def test_frame_loop_small(d):
    lay = small_layout(mask=True)
    q, k, v = qkv_random(1, 2, lay.n, d, seed=130 + d)
    kw = frame_loop(lay)
    assert kw["partitions"] == 7     # six target frames and the other rows
    check(q, k, v, lay, BIND, f"frame-loop binding d={d}", **kw)


def test_frame_loop_ranges_equal_and_empty_and_fp32():
    lay = small_layout(mask=True)
    q, k, v = qkv_random(1, 2, lay.n, 128, seed=133)
    check(q, k, v, lay, BIND, "frame-loop 5 near-equal ranges", mode="frame-loop", partitions=5)
    n = lay.n
    check(q, k, v, lay, BIND, "frame-loop with empty ranges", mode="frame-loop", partitions=4,
          bounds=[0, 0, 300, 300, n])
    qf, kf, vf = (x.float() for x in (q, k, v))
    check(qf, kf, vf, lay, BIND, "frame-loop fp32", **frame_loop(lay))


def test_frame_loop_shuffled_many_ranges():
    """A shuffled order cuts the rows into hundreds of short ranges."""
    base = small_layout(mask=True)
    lay = base.permuted(np.random.default_rng(134).permutation(base.n))
    q, k, v = qkv_random(1, 2, lay.n, 128, seed=135)
    kw = frame_loop(lay)
    log(f"shuffled frame loop: {kw['partitions']} ranges over {lay.n} rows")
    check(q, k, v, lay, BIND, "frame-loop shuffled", **kw)


@pytest.mark.parametrize("mode", ["dense-bias", "frame-loop"])
def test_baselines_fullsize_sampled(mode):
    """The benchmark workload (107,126 tokens x 56 heads, D 128), all heads in
    one call; stratified rows of three heads against the oracle, and the whole
    output against the fused mode."""
    cfg = ti.config(6)
    lay = cfg.layout()
    q, k, v = ti.qkv(cfg)
    heads = [0, cfg.heads // 2, cfg.heads - 1]
    rows = sample_rows(lay, n_random=128, per_segment=32, seed=140)
    kw = frame_loop(lay) if mode == "frame-loop" else dict(mode=mode)
    log(f"{mode}: N={lay.n} H={cfg.heads}")
    o, l = run_gpu(q, k, v, lay, cfg.params, heads=heads, rows=rows, **kw)
    ro, rl = run_oracle(q, k, v, lay, cfg.params, rows=rows, heads=heads)
    compare(o.numpy(), l.numpy(), ro, rl, what=f"{mode} config 6 sampled")
    of, lf = run_gpu(q, k, v, lay, cfg.params, heads=heads, rows=rows)
    dl, do = float((lf - l).abs().max()), float((of - o).abs().max())
    log(f"{mode} vs fused: max|dLSE|={dl:.3e} max|dO|={do:.3e}")
    assert dl <= 1e-3 and do <= 1e-2
