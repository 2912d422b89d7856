"""Out-of-range metadata, through the C ABI. By default such a token still
takes part in attention, nothing is read out of bounds, and it loses only the
term its bad field feeds: a segment code > 3 makes it an other token, a
picture id outside [0, num_pictures) removes its binding term, a non-finite
time takes a guide key out of the temporal term and a target query out of the
temporal term (the query keeps its binding term), and a non-finite mask weight
removes that query's binding term (its mask weight reads as 0). The result must
equal the oracle's on a layout that says the same with valid metadata: the
bad tokens turned into other tokens, except the target queries with a bad
time, whose rows are compared with the oracle run without the temporal term.
With TARA_VALIDATE=1 the same call is rejected with TARA_ERR_BAD_METADATA
before any work is enqueued.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import tara_inputs as ti
import temporally_biased_flashattention_amd as tara
from tara_testlib import compare, log, qkv_random, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

BIND = ti.Params(window=0.10, falloff=0.40, strength=3.0, cap=8.0, binding=True, gains=(1.25, 0.75, 0.6))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bad_layout():
    """A framed layout with bad metadata planted on a few tokens of every kind,
    and the same layout with those tokens turned into plain other tokens."""
    lay = ti.make_layout(6, (6, 10), (6, 10), 3, 40, 37, mask=True)
    rng = np.random.default_rng(31)
    seg, time, pic = lay.seg.copy(), lay.time.copy(), lay.picture.copy()
    tgt = np.nonzero(seg == ti.SEG_TARGET)[0]
    gd = np.nonzero(seg == ti.SEG_GUIDE)[0]
    pc = np.nonzero(seg == ti.SEG_PICTURE)[0]
    bad_seg = rng.choice(tgt, 4, replace=False)
    seg[bad_seg[:2]] = 5
    seg[bad_seg[2:]] = 200
    bad_time_t = rng.choice(np.setdiff1d(tgt, bad_seg), 3, replace=False)
    time[bad_time_t] = [np.nan, np.inf, -np.inf]
    bad_time_g = rng.choice(gd, 3, replace=False)
    time[bad_time_g] = [np.inf, np.nan, -np.inf]
    bad_pic = rng.choice(pc, 4, replace=False)
    pic[bad_pic] = [3, 40, -1, -7]          # num_pictures is 3
    bad_mask = rng.choice(np.setdiff1d(tgt, np.concatenate([bad_seg, bad_time_t])), 3, replace=False)
    mask = lay.mask.copy()
    mask[bad_mask] = [np.nan, np.inf, -np.inf]
    raw = ti.Layout(seg, time, pic, lay.frame, mask)
    clean_seg = seg.copy()
    clean_seg[np.concatenate([bad_seg, bad_time_g, bad_pic])] = ti.SEG_OTHER
    clean_time = time.copy()
    clean_time[clean_seg == ti.SEG_OTHER] = np.nan
    clean_time[bad_time_t] = 0.0          # their rows are checked without the temporal term
    clean_pic = pic.copy()
    clean_pic[clean_seg != ti.SEG_PICTURE] = -1
    clean_mask = mask.copy()
    clean_mask[bad_mask] = 0.0            # a non-finite weight drops that query's binding term
    clean = ti.Layout(clean_seg, clean_time, clean_pic, lay.frame, clean_mask)
    return raw, clean, bad_time_t


def _oracle(q, k, v, clean, bad_time_t, p):
    """The oracle on the valid layout; the target rows whose time was bad
    take the oracle without the temporal term (binding kept)."""
    ro, rl = run_oracle(q, k, v, clean, p)
    no_temporal = dataclasses.replace(p, strength=0.0)
    so, sl = run_oracle(q, k, v, clean, no_temporal, rows=np.sort(bad_time_t))
    ro[:, :, np.sort(bad_time_t)] = so
    rl[:, :, np.sort(bad_time_t)] = sl
    return ro, rl


@pytest.mark.parametrize("mode", ["fused", "three-term"])
def test_out_of_range_metadata_gets_no_bias(mode):
    raw, clean, bad_t = _bad_layout()
    q, k, v = qkv_random(1, 2, raw.n, 128, seed=32)
    o, l = run_gpu(q, k, v, raw, BIND, mode=mode)
    ro, rl = _oracle(q, k, v, clean, bad_t, BIND)
    compare(o.numpy(), l.numpy(), ro, rl, what=f"out-of-range metadata, {mode}")


def test_validate_rejects_out_of_range_metadata(monkeypatch):
    raw, clean, _ = _bad_layout()
    q, k, v = qkv_random(1, 1, raw.n, 64, seed=33)
    monkeypatch.setenv("TARA_VALIDATE", "1")
    with pytest.raises(tara.TaraError) as e:
        run_gpu(q, k, v, raw, BIND)
    log(f"TARA_VALIDATE=1 rejects: {e.value}")
    assert e.value.status == -8          # TARA_ERR_BAD_METADATA
    # the clean layout passes the same check and matches the oracle
    o, l = run_gpu(q, k, v, clean, BIND)
    ro, rl = run_oracle(q, k, v, clean, BIND)
    compare(o.numpy(), l.numpy(), ro, rl, what="TARA_VALIDATE=1, clean metadata")
    monkeypatch.delenv("TARA_VALIDATE")
    assert os.environ.get("TARA_VALIDATE") is None
