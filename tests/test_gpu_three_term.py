"""GPU parity of the three-term (Flash Partitions) mode: the library's three
term passes (keys that are not biased guide keys; guide keys with target rows
at -cap; the local correction inside the saturation gap), merged by LSE,
against the fp64 oracle's full attention, through the C ABI. Reading of the
"Three backends" section of "TARA: Native Temporal Alignment for MiniMax H3
References"; the oracle pins the split itself (P8). Same gates as the other
parity tests."""
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


def check(q, k, v, lay, p, what, **kw):
    o, l = run_gpu(q, k, v, lay, p, mode="three-term", **kw)
    ro, rl = run_oracle(q, k, v, lay, p)
    res = compare(o.numpy(), l.numpy(), ro, rl, what=what)
    of, lf = run_gpu(q, k, v, lay, p, **kw)
    dl = float((lf - l).abs().max())
    log(f"  three-term vs fused: max|dLSE|={dl:.3e} max|dO|={float((of - o).abs().max()):.3e}")
    assert dl <= 1e-3
    return res


@pytest.mark.parametrize("d", [128, 64])
def test_three_term_small(d):
    lay = ti.make_layout(6, (6, 10), (6, 10), 3, 40, 37, mask=True)
    q, k, v = qkv_random(1, 2, lay.n, d, seed=60 + d)
    check(q, k, v, lay, DEF, f"three-term defaults d={d}")
    check(q, k, v, lay, BIND, f"three-term binding d={d}")


def test_three_term_framed_chained_shuffled():
    lay = ti.make_layout(12, (8, 16), (8, 16), 3, 100, 50, mask=True, mask_planes=2)
    q, k, v = qkv_random(1, 2, lay.n, 128, seed=61)
    check(q, k, v, lay, CHAIN, "three-term framed chained")
    rng = np.random.default_rng(62)
    check(q, k, v, lay.permuted(rng.permutation(lay.n)), CHAIN, "three-term shuffled chained")


def test_three_term_fp32_and_degenerate():
    lay = ti.make_layout(6, (6, 10), (6, 10), 3, 40, 37, mask=True)
    q, k, v = qkv_random(1, 2, lay.n, 64, seed=63, dtype=torch.float32)
    check(q, k, v, lay, BIND, "three-term fp32")
    q, k, v = qkv_random(1, 2, lay.n, 128, seed=64)
    check(q, k, v, lay, ti.Params(strength=0.0), "three-term strength=0 (terms B, C empty)")
    check(q, k, v, lay, ti.Params(cap=0.0), "three-term cap=0")
    # a long free window: every guide key inside the window (constant correction class)
    check(q, k, v, lay, ti.Params(window=5.0), "three-term window covers every gap")


@pytest.mark.parametrize("n", [1, 65, 200, 700])
def test_three_term_ragged(n):
    rng = np.random.default_rng(200 + n)
    lay = ti.random_layout(rng, n, frames=4, pictures=2, mask=True)
    q, k, v = qkv_random(1, 2, n, 128, seed=65 + n)
    check(q, k, v, lay, ti.Params(binding=True, gains=(1.5, 0.6)), f"three-term n={n}")


def test_three_term_segment_extremes():
    n = 700
    q, k, v = qkv_random(1, 2, n, 128, seed=66)
    for name, seg in (("all target", ti.SEG_TARGET), ("all guide", ti.SEG_GUIDE)):
        lay = ti.make_layout(7, (10, 10), (0, 0), 0, 0, 0)
        lay.seg[:] = seg
        check(q, k, v, lay, DEF, f"three-term {name}")


@pytest.mark.parametrize("cid", [5, 6])
def test_fullsize_three_term_sampled_rows(cid):
    """Full sequence length, two heads; the outputs are NaN-poisoned before
    the call and every element must be written (by the merge of the three
    term partitions)."""
    cfg = ti.config(cid)
    lay = cfg.layout()
    q, k, v = ti.qkv(cfg, heads=[0, 1])
    rows = sample_rows(lay, n_random=256, per_segment=64, seed=80 + cid)
    log(f"config {cid}: N={lay.n}, three-term, {len(rows)} rows x 2 heads")
    o, l = run_gpu(q, k, v, lay, cfg.params, mode="three-term", rows=rows, poison=True)
    ro, rl = run_oracle(q, k, v, lay, cfg.params, rows=rows)
    compare(o.numpy(), l.numpy(), ro, rl, what=f"config {cid} three-term sampled")
