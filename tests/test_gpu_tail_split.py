"""Fused bf16 calls whose workgroups would leave the chip's last round of
compute units partly filled: the first query blocks of every head run as the
fused pass, the rest as the range pass over a few key ranges plus the exact
LSE merge of those rows. At 20,020 tokens x 8 heads (79 query blocks per head
of 256 rows: 632 workgroups, 2.5 rounds of 256) rows 0..16,383 take the fused
pass and rows 16,384.. two key ranges. Rows on both sides of that boundary,
and the last rows, are checked against the oracle with the parity gates, on
poisoned outputs; the call is checked against the partitioned mode, and its
run info shows the extra launches."""
import numpy as np
import pytest
import torch

import tara_inputs as ti
import temporally_biased_flashattention_amd as tara
from tara_testlib import compare, log, qkv_random, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _layout():
    # 20 latent frames of 17 x 29 target and guide patches, 2 pictures of 100
    # tokens, 100 text tokens: 20,020 tokens
    return ti.make_layout(frames=20, target_hw=(17, 29), guide_hw=(17, 29), pictures=2,
                          picture_tokens=100, text=100)


@pytest.mark.parametrize("d,B", [(128, 1), (64, 1), (128, 2)])
def test_tail_split_rows(d, B):
    """8 (batch, head) pairs: 1 x 8 heads, or 2 batch elements x 4 heads."""
    lay = _layout()
    n = lay.n
    assert n == 20020
    H = 8 // B
    split_row = 64 * 256
    q, k, v = qkv_random(B, H, n, d, seed=7700 + d + B)
    p = ti.Params()
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([
        np.arange(split_row - 40, split_row + 40),            # both sides of the split
        np.arange(n - 40, n),                                 # the last rows
        rng.choice(split_row, size=60, replace=False),        # fused-pass rows
        rng.integers(split_row, n, size=60),                  # split-off rows
    ]))
    o, l = run_gpu(q, k, v, lay, p, rows=rows, poison=True)
    info = tara.tara_get_last_run_info()
    log(f"D={d} B={B}: run info {info}")
    # meta, V^T, key norms, the fused pass, the range pass over the split-off rows, their merge
    assert info["launches"] == 6 and info["tail_parts"] == 2
    assert info["grid"] == B * H * 64 + B * H * 15 * 2
    ro, rl = run_oracle(q, k, v, lay, p, rows=rows)
    compare(o.numpy(), l.numpy(), ro, rl, what=f"tail split D={d}, B={B}, {len(rows)} rows x {H} heads")
    # the partitioned mode over the same rows agrees to rounding
    po, pl = run_gpu(q, k, v, lay, p, mode="partitioned", partitions=3, rows=rows)
    dl = float((pl - l).abs().max())
    do = float((po - o).abs().max())
    log(f"fused (tail split) vs partitioned: max|dLSE|={dl:.3e} max|dO|={do:.3e}")
    assert dl <= 1e-4 and do <= 2e-2


def test_no_split_below_one_round():
    """A call within one round of workgroups (here 8 x 4 = 32) runs as one
    fused pass: meta, V^T, key norms, attention."""
    lay = ti.make_layout(frames=2, target_hw=(17, 29), guide_hw=(17, 29), pictures=1, picture_tokens=20, text=8)
    q, k, v = qkv_random(1, 8, lay.n, 128, seed=7800)
    run_gpu(q, k, v, lay, ti.Params(), rows=np.arange(lay.n))
    assert tara.tara_get_last_run_info()["launches"] == 4


def test_tail_split_qk8():
    """8-bit Q.K: the range pass of the tail takes FP8 products too. Rows on
    both sides of the split and the last rows against the oracle run on the
    dequantised Q and K (the usual gates)."""
    from tara_testlib import dequantized
    lay = _layout()
    n = lay.n
    H, d = 8, 128
    split_row = 64 * 256
    q, k, v = qkv_random(1, H, n, d, seed=7900)
    rows = np.unique(np.concatenate([np.arange(split_row - 24, split_row + 24), np.arange(n - 24, n)]))
    o, l = run_gpu(q, k, v, lay, ti.Params(), qk8=True, rows=rows, poison=True)
    info = tara.tara_get_last_run_info()
    assert info["tail_parts"] == 2 and info["launches"] == 6, info
    hs = list(range(H))
    qd, kd = dequantized(q, k, heads=hs, rows=rows)
    ro, rl = run_oracle(qd, kd, v, lay, ti.Params(), rows=rows, heads=hs)
    compare(o.numpy(), l.numpy(), ro, rl, what=f"tail split 8-bit Q.K, {len(rows)} rows x {H} heads")
