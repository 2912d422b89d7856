"""GPU parity of chained reference bindings ("BFS H3 Reference Attention
Binding (Experimental)", section "Common issues": chained binding nodes add
their log gains, sum_j m_j * ln(gain_j,i)) against the fp64 oracle, through
the C ABI. Same gates as the other parity tests."""
import numpy as np
import pytest
import torch

import tara_inputs as ti
from tara_testlib import compare, log, qkv_random, run_gpu, run_oracle, sample_rows

pytestmark = pytest.mark.gpu

G1 = (1.25, 0.75, 0.75)
G2 = (0.8, 1.4, 1.1)
G3 = (1.6, 0.5, 2.0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def planes_layout(nplanes, frames=6, hw=(6, 10), pictures=3, ptok=40, text=37):
    return ti.make_layout(frames, hw, hw, pictures, ptok, text, mask=True, mask_planes=nplanes)


def params(*gain_sets, **kw):
    p = dict(window=0.10, falloff=0.40, strength=3.0, cap=8.0)
    p.update(kw)
    return ti.Params(**p, binding=True, gains=gain_sets[0], chained=tuple(gain_sets[1:]))


def check(q, k, v, lay, p, what, **kw):
    o, l = run_gpu(q, k, v, lay, p, **kw)
    ro, rl = run_oracle(q, k, v, lay, p, use_mask=kw.get("use_mask", True))
    return compare(o.numpy(), l.numpy(), ro, rl, what=what)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("nb", [2, 3])
def test_chained_small(d, nb):
    lay = planes_layout(nb)
    q, k, v = qkv_random(1, 2, lay.n, d, seed=40 + nb + d)
    p = params(*(G1, G2, G3)[:nb])
    check(q, k, v, lay, p, f"{nb} bindings d={d}")
    check(q, k, v, lay, p, f"{nb} bindings no mask d={d}", use_mask=False)


def test_chained_framed_and_shuffled():
    lay = ti.make_layout(12, (8, 16), (8, 16), 3, 100, 50, mask=True, mask_planes=2)
    q, k, v = qkv_random(1, 2, lay.n, 128, seed=50)
    check(q, k, v, lay, params(G1, G2), "framed 2 bindings")
    rng = np.random.default_rng(51)
    sh = lay.permuted(rng.permutation(lay.n))
    check(q, k, v, sh, params(G1, G2), "shuffled 2 bindings")


def test_chained_fp32_and_partitioned():
    lay = planes_layout(2)
    q, k, v = qkv_random(1, 2, lay.n, 64, seed=52, dtype=torch.float32)
    check(q, k, v, lay, params(G1, G2), "fp32 2 bindings")
    q, k, v = qkv_random(1, 2, lay.n, 128, seed=53)
    check(q, k, v, lay, params(G1, G2), "partitioned 2 bindings", mode="partitioned", partitions=4)


def test_equal_masks_equal_product_gains_on_gpu():
    """Two bindings sharing one mask plane give the same logits as one binding
    whose gains are the products (log gains add); GPU against GPU."""
    base = planes_layout(1)
    two = ti.Layout(base.seg, base.time, base.picture, base.frame, np.stack([base.mask, base.mask]))
    q, k, v = qkv_random(1, 2, base.n, 128, seed=54)
    o2, l2 = run_gpu(q, k, v, two, params(G1, G2))
    o1, l1 = run_gpu(q, k, v, base, params(tuple(a * b for a, b in zip(G1, G2))))
    dl, do = float((l2 - l1).abs().max()), float((o2 - o1).abs().max())
    log(f"chained vs product gains: max|dLSE|={dl:.3e} max|dO|={do:.3e}")
    assert dl <= 1e-4 and do <= 1e-2


def test_fullsize_chained_sampled_rows():
    cfg = ti.config(7)
    lay = cfg.layout()
    q, k, v = ti.qkv(cfg, heads=[0, 1])
    rows = sample_rows(lay, n_random=256, per_segment=64, seed=77)
    log(f"config 7 {cfg.name}: N={lay.n}, {len(rows)} rows x 2 heads")
    o, l = run_gpu(q, k, v, lay, cfg.params, rows=rows)
    ro, rl = run_oracle(q, k, v, lay, cfg.params, rows=rows)
    compare(o.numpy(), l.numpy(), ro, rl, what="config 7 chained bindings sampled")
