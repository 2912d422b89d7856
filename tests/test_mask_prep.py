"""Host preparation of the per-token mask weight from a soft pixel mask.

The binding page ("BFS H3 Reference Attention Binding (Experimental)") fixes:
a mask is one frame or exactly the prepared 17n + 5 shot length, anything else
throws ("Common issues"); soft masks are area-downsampled to the target patch
resolution and averaged over the latent temporal spans ("The exact rule"); no
mask means the gain applies to every output position ("Inputs you'll set").
CPU only.
"""
import pathlib

import numpy as np
import pytest

import tara_inputs as ti
from oracle import tara_oracle as oracle

GOLDEN = pathlib.Path(__file__).parent / "golden" / "mask_area_downsample.txt"


def _golden():
    out = {}
    for line in GOLDEN.read_text().splitlines():
        if line.startswith("#") or not line.strip():
            continue
        key, *vals = line.split()
        out[key] = np.array([float(v) for v in vals])
    return out


@pytest.mark.parametrize("frames", [5, 22, 39, 90, 107, 5 + 17 * 20])
def test_shot_lengths_accepted(frames):
    assert ti.shot_length_ok(frames)
    m = np.full((frames, 4, 4), 0.5)
    out = ti.prepare_target_mask(m, frames, 3, (2, 2))
    assert out.shape == (12,) and np.allclose(out, 0.5)


@pytest.mark.parametrize("frames", [0, 1, 2, 4, 6, 21, 23, 106, 108])
def test_bad_shot_lengths_rejected(frames):
    assert not ti.shot_length_ok(frames)
    with pytest.raises(ValueError, match="17n"):
        ti.prepare_target_mask(np.ones((1, 4, 4)), frames, 3, (2, 2))


def test_mask_length_mismatch_throws():
    # a whole-clip mask into a 107-frame shot, and one frame short of it
    for f in (200, 106, 2):
        with pytest.raises(ValueError, match="mask length"):
            ti.prepare_target_mask(np.ones((f, 4, 4)), 107, 27, (2, 2))
    # one frame, or a [height, width] array, is the static mask
    a = ti.prepare_target_mask(np.ones((1, 4, 4)), 107, 27, (2, 2))
    b = ti.prepare_target_mask(np.ones((4, 4)), 107, 27, (2, 2))
    assert np.array_equal(a, b)


def test_non_finite_mask_rejected():
    m = np.ones((1, 4, 4))
    m[0, 1, 2] = np.nan
    with pytest.raises(ValueError, match="finite"):
        ti.prepare_target_mask(m, 22, 5, (2, 2))


def test_hand_worked_cases():
    g = _golden()
    out1 = ti.prepare_target_mask(g["case1_mask"].reshape(3, 3), 5, 1, (2, 2))
    assert np.allclose(out1, g["case1_out"], rtol=0, atol=1e-7)
    frames = np.stack([np.full((2, 2), f / 4.0) for f in range(5)])
    out2 = ti.prepare_target_mask(frames, 5, 2, (1, 1))
    assert np.allclose(out2, g["case2_out"], rtol=0, atol=1e-7)


def test_block_mean_when_sizes_divide():
    # an exact block mean (reshape), independent of the overlap weights
    rng = np.random.default_rng(3)
    T, k, rows, cols, a, b = 4, 1, 3, 5, 4, 2
    shot = 22
    m = rng.uniform(size=(shot, rows * a, cols * b))
    out = ti.prepare_target_mask(m, shot, T, (rows, cols)).reshape(T, rows, cols)
    blocks = m.reshape(shot, rows, a, cols, b).mean(axis=(2, 4))
    for j, (lo, hi) in enumerate(ti.latent_spans(shot, T)):
        assert np.allclose(out[j], blocks[lo:hi].mean(axis=0), rtol=0, atol=1e-6)


def test_mean_is_kept_for_any_sizes():
    # equal-area cells: each latent frame's mean over the patches equals the
    # mean of its span's pixels, whatever the sizes
    rng = np.random.default_rng(4)
    shot, T = 39, 7
    m = rng.uniform(size=(shot, 17, 23))
    out = ti.prepare_target_mask(m, shot, T, (5, 6)).reshape(T, 5, 6)
    for j, (lo, hi) in enumerate(ti.latent_spans(shot, T)):
        assert abs(out[j].mean() - m[lo:hi].mean()) < 1e-6


def test_spans_cover_the_shot():
    for frames, T in ((107, 27), (22, 6), (5, 2), (5, 9), (1, 4)):
        spans = ti.latent_spans(frames, T)
        assert len(spans) == T and all(0 <= lo < hi <= frames for lo, hi in spans)
        if frames >= T:
            # consecutive, disjoint, covering every frame once
            assert spans[0][0] == 0 and spans[-1][1] == frames
            assert all(spans[i][1] == spans[i + 1][0] for i in range(T - 1))


def test_static_mask_same_on_every_latent_frame():
    rng = np.random.default_rng(5)
    m = rng.uniform(size=(9, 14))
    out = ti.prepare_target_mask(m, 107, 27, (3, 4)).reshape(27, 12)
    assert np.array_equal(out, np.broadcast_to(out[0], out.shape))


def test_all_ones_mask_equals_no_mask_in_the_oracle():
    # m = 1 on every target token is what no mask means: the oracle's output is
    # the same with the prepared all-ones mask and with no mask
    frames, rows, cols = 3, 2, 2
    lay = ti.make_layout(frames, (rows, cols), (rows, cols), 2, 4, 6)
    n = lay.n
    nt = frames * rows * cols
    m = np.zeros(n, np.float32)
    m[:nt] = ti.prepare_target_mask(np.ones((22, 8, 8)), 22, frames, (rows, cols))
    p = ti.Params(binding=True, gains=(1.25, 0.75))
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((n, 16)) for _ in range(3))
    o1, l1 = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, m, p)
    o2, l2 = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, None, p)
    # and a half-weight mask moves the output (the mask is read)
    o3, _ = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, 0.5 * m, p)
    assert np.abs(o3 - o1).max() > 1e-3
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)
