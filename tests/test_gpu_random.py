"""Randomised GPU parity sweep against the fp64 oracle, through the C ABI.

Each seeded case draws a sequence with all four segment kinds in random
proportions (shuffled or in order), random latent-frame times, picture ids
and mask weights; random valid controls (window, falloff, strength, cap,
binding gains, up to four chained bindings with their own mask planes); a
length from 1 to ~2,600 tokens; head dim 64 or 128; bf16 or fp32; and one of
the modes (fused, partitioned with random key bounds, three-term, frame-loop
with random query ranges, dense-bias, 8-bit Q.K). Gates as everywhere:
max|dO| <= 1e-2, max|dLSE| <= 1e-3, relative 1e-2; the 8-bit mode is
compared with the oracle run on its rounded Q and K.
"""
import dataclasses

import numpy as np
import pytest
import torch

import tara_inputs as ti
from tara_testlib import compare, dequantized, log, qkv_random, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

NCASES = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bounds(rng, n, parts):
    inner = np.sort(rng.integers(0, n + 1, size=parts - 1)) if parts > 1 else np.array([], np.int64)
    return [0] + [int(x) for x in inner] + [n]


def make_case(seed):
    rng = np.random.default_rng(7000 + seed)
    band = int(rng.integers(0, 3))
    n = int(rng.integers(1, 130) if band == 0 else rng.integers(130, 1200) if band == 1 else rng.integers(1200, 2600))
    d = int(rng.choice([64, 128]))
    heads = int(rng.integers(1, 3))
    pictures = int(rng.integers(1, 6))
    use_mask = bool(rng.integers(0, 2))
    lay = ti.random_layout(rng, n, frames=int(rng.integers(1, 10)), pictures=pictures, mask=use_mask,
                           shuffle=bool(rng.integers(0, 2)))
    p = ti.random_params(rng, pictures)
    if p.binding and rng.integers(0, 2):
        nb = int(rng.integers(2, 5))
        chained = tuple(tuple(float(x) for x in rng.uniform(0.3, 2.5, size=pictures)) for _ in range(nb - 1))
        p = dataclasses.replace(p, chained=chained)
        if lay.mask is not None:
            planes = [lay.mask]
            tgt = lay.seg == ti.SEG_TARGET
            for _ in range(nb - 1):
                m = np.zeros(n, np.float32)
                m[tgt] = rng.uniform(0.0, 1.0, size=int(tgt.sum())).astype(np.float32)
                planes.append(m)
            lay = ti.Layout(lay.seg, lay.time, lay.picture, lay.frame, np.stack(planes))
    fp32 = rng.random() < 0.2
    modes = ["fused", "partitioned", "three-term", "frame-loop"] + ([] if fp32 else ["dense-bias", "qk8"])
    mode = str(rng.choice(modes))
    kw = {}
    if mode == "partitioned":
        parts = int(rng.integers(1, 7))
        kw = dict(mode="partitioned", partitions=parts, bounds=_bounds(rng, n, parts) if rng.integers(0, 2) else None)
    elif mode == "frame-loop":
        parts = int(rng.integers(1, min(n, 12) + 1))
        kw = dict(mode="frame-loop", partitions=parts, bounds=_bounds(rng, n, parts))
    elif mode == "qk8":
        kw = dict(qk8=True)
    elif mode != "fused":
        kw = dict(mode=mode)
    return dict(n=n, d=d, heads=heads, lay=lay, p=p, fp32=fp32, mode=mode, kw=kw, seed=seed)


@pytest.mark.parametrize("seed", range(NCASES))
def test_random_case(seed):
    c = make_case(seed)
    lay, p = c["lay"], c["p"]
    what = (f"seed {seed}: n={c['n']} d={c['d']} H={c['heads']} {'fp32' if c['fp32'] else 'bf16'} {c['mode']} "
            f"binding={p.binding} bindings={1 + len(p.chained)} mask={lay.mask is not None} "
            f"s={p.strength:.2f} cap={p.cap:.2f} w={p.window:.2f} f={p.falloff:.2f}")
    log(what)
    q, k, v = qkv_random(1, c["heads"], c["n"], c["d"], seed=8000 + seed,
                         dtype=torch.float32 if c["fp32"] else torch.bfloat16)
    o, l = run_gpu(q, k, v, lay, p, **c["kw"])
    if c["mode"] == "qk8":
        q, k = dequantized(q, k)
    ro, rl = run_oracle(q, k, v, lay, p)
    compare(o.numpy(), l.numpy(), ro, rl, what=what)
