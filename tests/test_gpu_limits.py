"""GPU parity at the library's stated limits, through the C ABI, against the
fp64 oracle: the most pictures (16) with the most chained bindings (4, each
with its own gains and mask plane), the most caller partitions (64, some of
them empty), a frame loop with one launch per query row, and a three-term
call at the longest sequence its per-workgroup tile list holds (2^20 tokens,
16,384 key tiles). Same gates as the other parity tests.
"""
import dataclasses

import numpy as np
import pytest
import torch

import tara_inputs as ti
from tara_testlib import compare, log, qkv_random, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

MAX_PICTURES = 16
MAX_BINDINGS = 4
MAX_PARTITIONS = 64
MAX_THREE_TERM_N = 1 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _max_binding_case(seed, n):
    """Shuffled layout (40% target, 30% guide, 20% pictures, the rest text)
    whose picture tokens carry all 16 ids, binding on, 4 bindings with their
    own gains (one per picture) and mask planes."""
    rng = np.random.default_rng(seed)
    counts = [int(0.4 * n), int(0.3 * n), int(0.2 * n)]
    counts.append(n - sum(counts))
    seg = np.repeat(np.arange(4, dtype=np.uint8), counts)
    frame = np.full(n, -1, np.int32)
    vid = seg <= ti.SEG_GUIDE
    frame[vid] = rng.integers(0, 8, size=int(vid.sum()))
    time = np.full(n, np.nan, np.float32)
    time[vid] = ti.frame_time(frame[vid])
    pic = np.full(n, -1, np.int16)
    isp = seg == ti.SEG_PICTURE
    pic[isp] = (np.arange(int(isp.sum())) % MAX_PICTURES).astype(np.int16)
    mask = np.zeros(n, np.float32)
    mask[seg == ti.SEG_TARGET] = rng.uniform(0.0, 1.0, size=counts[0]).astype(np.float32)
    lay = ti.Layout(seg, time, pic, frame, mask).permuted(rng.permutation(n))
    p = ti.random_params(rng, MAX_PICTURES, binding=True)
    p = dataclasses.replace(p, strength=max(p.strength, 1.0), cap=max(p.cap, 2.0))
    chained = tuple(tuple(float(x) for x in rng.uniform(0.3, 2.5, size=MAX_PICTURES))
                    for _ in range(MAX_BINDINGS - 1))
    p = dataclasses.replace(p, chained=chained)
    planes = [lay.mask]
    tgt = lay.seg == ti.SEG_TARGET
    for _ in range(MAX_BINDINGS - 1):
        m = np.zeros(n, np.float32)
        m[tgt] = rng.uniform(0.0, 1.0, size=int(tgt.sum())).astype(np.float32)
        planes.append(m)
    lay = ti.Layout(lay.seg, lay.time, lay.picture, lay.frame, np.stack(planes))
    return lay, p


@pytest.mark.parametrize("mode", ["fused", "three-term"])
@pytest.mark.parametrize("d", [128, 64])
def test_max_pictures_and_bindings(d, mode):
    lay, p = _max_binding_case(9100 + d, 1400)
    assert len(p.gains) == MAX_PICTURES and 1 + len(p.chained) == MAX_BINDINGS
    assert int(lay.picture.max()) == MAX_PICTURES - 1
    q, k, v = qkv_random(1, 2, lay.n, d, seed=9200 + d)
    what = f"16 pictures x 4 bindings, d={d}, {mode}"
    log(what)
    o, l = run_gpu(q, k, v, lay, p, mode=mode)
    ro, rl = run_oracle(q, k, v, lay, p)
    compare(o.numpy(), l.numpy(), ro, rl, what=what)


def test_max_pictures_and_bindings_fp32():
    lay, p = _max_binding_case(9300, 900)
    q, k, v = qkv_random(1, 1, lay.n, 64, seed=9301, dtype=torch.float32)
    o, l = run_gpu(q, k, v, lay, p)
    ro, rl = run_oracle(q, k, v, lay, p)
    compare(o.numpy(), l.numpy(), ro, rl, what="16 pictures x 4 bindings, fp32")


@pytest.mark.parametrize("bounds", ["even", "ragged"])
def test_max_partitions(bounds):
    """64 key ranges (the most a call takes), merged exactly; the ragged split
    has empty ranges and ranges that cut key tiles."""
    rng = np.random.default_rng(9400)
    n = 1500
    lay = ti.random_layout(rng, n, frames=10, pictures=3, mask=True, shuffle=True)
    p = ti.random_params(rng, 3, binding=True)
    b = None
    if bounds == "ragged":
        inner = np.sort(rng.integers(0, n + 1, size=MAX_PARTITIONS - 1))
        inner[5] = inner[4]            # at least one empty range
        b = [0] + [int(x) for x in inner] + [n]
    q, k, v = qkv_random(1, 2, n, 128, seed=9401)
    what = f"{MAX_PARTITIONS} partitions ({bounds})"
    log(what)
    o, l = run_gpu(q, k, v, lay, p, mode="partitioned", partitions=MAX_PARTITIONS, bounds=b)
    ro, rl = run_oracle(q, k, v, lay, p)
    compare(o.numpy(), l.numpy(), ro, rl, what=what)


def test_frame_loop_one_row_per_range():
    """The frame-loop baseline with one launch per query row."""
    rng = np.random.default_rng(9500)
    n = 300
    lay = ti.random_layout(rng, n, frames=6, pictures=2, mask=True, shuffle=False)
    p = ti.random_params(rng, 2)
    q, k, v = qkv_random(1, 1, n, 64, seed=9501)
    o, l = run_gpu(q, k, v, lay, p, mode="frame-loop", partitions=n, bounds=list(range(n + 1)))
    ro, rl = run_oracle(q, k, v, lay, p)
    compare(o.numpy(), l.numpy(), ro, rl, what=f"frame loop, {n} one-row ranges")


def _longest_three_term_layout():
    # 512 latent frames of 32 x 32 target and 31 x 32 guide patches, two
    # pictures of 7,168 tokens and 2,048 text tokens: exactly 2^20 tokens
    lay = ti.make_layout(frames=512, target_hw=(32, 32), guide_hw=(31, 32), pictures=2,
                         picture_tokens=7168, text=2048)
    assert lay.n == MAX_THREE_TERM_N
    return lay


@pytest.mark.timeout(300)
def test_three_term_at_longest_sequence():
    """2^20 tokens (16,384 key tiles, the most a term pass can list): the
    three-term result equals the fused one on every row, and both match the
    oracle on sampled rows."""
    lay = _longest_three_term_layout()
    p = ti.Params()
    q, k, v = qkv_random(1, 1, lay.n, 64, seed=9600)
    log(f"N={lay.n}: three-term and fused, all rows")
    ot, lt = run_gpu(q, k, v, lay, p, mode="three-term")
    of, lf = run_gpu(q, k, v, lay, p)
    dl = float((lt - lf).abs().max())
    do = float((ot - of).abs().max())
    log(f"three-term vs fused over all {lay.n} rows: max|dLSE|={dl:.3e} max|dO|={do:.3e}")
    assert torch.isfinite(lt).all() and torch.isfinite(ot).all()
    assert dl <= 1e-3 and do <= 1e-2
    rng = np.random.default_rng(9601)
    tgt = np.nonzero(lay.seg == ti.SEG_TARGET)[0]
    rows = set(int(x) for x in rng.choice(tgt, size=24, replace=False))
    for s in (ti.SEG_GUIDE, ti.SEG_PICTURE, ti.SEG_OTHER):
        idx = np.nonzero(lay.seg == s)[0]
        rows.update(int(x) for x in rng.choice(idx, size=4, replace=False))
    rows.update([0, int(tgt[-1]), lay.n - 1])
    rows = np.array(sorted(rows), dtype=np.int64)
    log(f"oracle on {rows.size} rows against all {lay.n} keys")
    ro, rl = run_oracle(q, k, v, lay, p, rows=rows)
    ri = torch.as_tensor(rows)
    compare(ot[:, :, ri].numpy(), lt[:, :, ri].numpy(), ro, rl, what=f"three-term N={lay.n}, {rows.size} rows")
