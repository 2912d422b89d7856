"""Pins of the fp64 oracle against what the TARA pages and mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
closed forms (tests/golden/penalty_closed_form.txt), the article's printed
"about 0.633 s", textbook attention from torch's own routine, brute force,
exact identities and invariances. test_pins_catch_planted_mistakes plants
plausible mistakes in the oracle (on the CPU) and checks that a pin fails.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.tara_oracle as tor
import tara_inputs as ti


# ------------------------------------------------------------------ fixtures
def _load_penalty_fixture(golden_dir):
    rows, sats = [], {}
    with open(os.path.join(golden_dir, "penalty_closed_form.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            p = line.split()
            if p[0] == "sat":
                sats[p[1]] = float(p[2])
            else:
                rows.append(dict(set=p[0], window=float(p[1]), falloff=float(p[2]),
                                 strength=float(p[3]), cap=float(p[4]), df=int(p[5]),
                                 value=Fraction(int(p[6]), int(p[7]))))
    return rows, sats


@pytest.fixture(scope="module")
def penalty_fixture(golden_dir):
    return _load_penalty_fixture(golden_dir)


DEFAULTS = ti.Params()
BIND5 = ti.Params(window=0.10, falloff=0.40, strength=3.0, cap=8.0, binding=True,
                  gains=(1.25, 0.75, 0.75))


# ------------------------------------------------------------------ P1: closed form
def test_p1_penalty_closed_form(penalty_fixture):
    rows, _ = penalty_fixture
    assert len(rows) >= 12
    for r in rows:
        got = tor.penalty(r["df"] * 4.0 / 24.0, r["window"], r["falloff"], r["strength"], r["cap"])
        assert abs(float(got) - float(r["value"])) < 1e-12, r


def test_p1_saturation_gap_matches_article(penalty_fixture):
    _, sats = penalty_fixture
    d = tor.saturation_gap(0.20, 0.25, 2.0, 6.0)
    assert abs(d - 0.633) < 5e-4               # the article's "about 0.633 s"
    assert abs(d - sats["defaults"]) < 1e-15
    assert abs(tor.saturation_gap(0.10, 0.40, 3.0, 8.0) - sats["binding"]) < 1e-15
    for p in (DEFAULTS, BIND5):
        g = tor.saturation_gap(p.window, p.falloff, p.strength, p.cap)
        # exactly the cap at the gap, strictly below just before it, the cap beyond
        assert abs(tor.penalty(g, p.window, p.falloff, p.strength, p.cap) - p.cap) < 1e-12
        assert tor.penalty(g - 1e-6, p.window, p.falloff, p.strength, p.cap) < p.cap
        far = np.linspace(g + 1e-9, g + 30.0, 1001)
        assert np.all(tor.penalty(far, p.window, p.falloff, p.strength, p.cap) == p.cap)


def test_p1_free_window_and_shape():
    p = DEFAULTS
    inside = np.linspace(0.0, p.window, 2001)
    assert np.all(tor.penalty(inside, p.window, p.falloff, p.strength, p.cap) == 0.0)
    assert np.all(tor.penalty(-inside, p.window, p.falloff, p.strength, p.cap) == 0.0)
    dt = np.linspace(0.0, 2.0, 4001)
    y = tor.penalty(dt, p.window, p.falloff, p.strength, p.cap)
    assert np.all(np.diff(y) >= 0.0)                       # grows with the gap
    assert np.all(y <= p.cap) and np.all(y >= 0.0)
    # quadratic growth past the window: second differences constant until the cap
    g = tor.saturation_gap(p.window, p.falloff, p.strength, p.cap)
    x = np.linspace(p.window + 0.01, g - 0.01, 50)
    yy = tor.penalty(x, p.window, p.falloff, p.strength, p.cap)
    h = x[1] - x[0]
    assert np.allclose(np.diff(yy, 2) / h ** 2, 2 * p.strength / p.falloff ** 2, rtol=1e-6)


# ------------------------------------------------- P2: reduces to textbook attention
def _torch_sdpa(q, k, v):
    qt, kt, vt = (torch.from_numpy(np.asarray(x, np.float64)) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None])[0]
    lse = torch.logsumexp(qt @ kt.T / math.sqrt(qt.shape[-1]), dim=-1)
    return o.numpy(), lse.numpy()


@pytest.mark.parametrize("case", ["strength0", "cap0", "wide_window", "no_target"])
def test_p2_reduces_to_sdpa(case):
    rng = np.random.default_rng(7)
    lay = ti.make_layout(6, (4, 4), (4, 4), 1, 16, 32)
    n, d = lay.n, 32
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    p = ti.Params()
    seg = lay.seg.copy()
    if case == "strength0":
        p = ti.Params(strength=0.0)
    elif case == "cap0":
        p = ti.Params(cap=0.0)
    elif case == "wide_window":
        p = ti.Params(window=10.0)
    else:
        seg[seg == ti.SEG_TARGET] = ti.SEG_OTHER
    o, lse = oracle.attention_head(q, k, v, seg, lay.time, lay.picture, None, p)
    ro, rl = _torch_sdpa(q, k, v)
    assert np.max(np.abs(o - ro)) < 1e-12
    assert np.max(np.abs(lse - rl)) < 1e-12
    # and the default rule does differ on the same data (the pin is not vacuous)
    o2, lse2 = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, None, ti.Params())
    assert np.max(np.abs(lse2 - rl)) > 0.1


# ------------------------------------------------------- P3: neutral binding
def test_p3_neutral_binding_bit_identical():
    rng = np.random.default_rng(11)
    lay = ti.make_layout(4, (3, 4), (3, 4), 3, 10, 9, mask=True)
    n, d = lay.n, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    base = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, lay.mask, ti.Params())
    variants = [
        ti.Params(binding=True, gains=(1.0, 1.0, 1.0)),                       # gain 1 is neutral
        ti.Params(binding=False, gains=(1.25, 0.75, 0.75)),                   # enabled off
    ]
    for p in variants:
        o, l = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, lay.mask, p)
        assert np.array_equal(o, base[0]) and np.array_equal(l, base[1])
    zero_m = np.zeros_like(lay.mask)
    o, l = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, zero_m,
                                 ti.Params(binding=True, gains=(1.25, 0.75, 0.75)))
    assert np.array_equal(o, base[0]) and np.array_equal(l, base[1])


# ------------------------------------------------------- P4: Q = 0 closed form
def _q0_expected(lay, pen_by_df, gains=None, m=1.0):
    """LSE and guide/picture mass of a target row in each frame when all Q.K = 0.

    Every unbiased key contributes e^0 = 1; a guide key df frames away
    contributes e^{-penalty(df)} with the hand-worked penalty; a picture key of
    id i contributes gain_i^m. Built from token counts only.
    """
    seg, frame, pic = lay.seg, lay.frame, lay.picture
    frames = int(frame.max()) + 1
    guide_per_frame = np.bincount(frame[seg == ti.SEG_GUIDE], minlength=frames)
    n_plain = int(np.sum((seg == ti.SEG_TARGET) | (seg == ti.SEG_OTHER)))
    pics = pic[seg == ti.SEG_PICTURE]
    out = {}
    for f in range(frames):
        guide = sum(float(guide_per_frame[g]) * math.exp(-float(pen_by_df[abs(f - g)]))
                    for g in range(frames))
        if gains is None:
            picture = float(len(pics))
        else:
            picture = sum(float(gains[int(i)]) ** m for i in pics)
        z = n_plain + guide + picture
        out[f] = (math.log(z), guide / z, picture / z)
    return out


def _exact_time(lay):
    """Token times df / 6 s in fp64 (the closed forms use exact gaps)."""
    return np.where(lay.frame >= 0, lay.frame * 4.0 / 24.0, np.nan)


def _probe_v(lay):
    v = np.zeros((lay.n, 4))
    v[lay.seg == ti.SEG_GUIDE, 0] = 1.0
    v[lay.seg == ti.SEG_PICTURE, 1] = 1.0
    v[:, 2] = 1.0
    return v


@pytest.mark.parametrize("which", ["defaults", "binding"])
def test_p4_q0_closed_form(penalty_fixture, which):
    rows, _ = penalty_fixture
    table = {r["df"]: r["value"] for r in rows if r["set"] == which}
    p = DEFAULTS if which == "defaults" else BIND5
    cap = Fraction(p.cap).limit_denominator(1000)
    pen_by_df = {df: table.get(df, cap if df >= 5 else None) for df in range(0, 40)}
    assert all(v is not None for v in pen_by_df.values())
    lay = ti.make_layout(6, (4, 4), (4, 4), 3 if which == "binding" else 1, 16, 32)
    n = lay.n
    q = np.zeros((n, 8))
    k = np.random.default_rng(3).standard_normal((n, 8))
    v = _probe_v(lay)
    for gains, m in ([None, 1.0], [(1.25, 0.75, 0.75), 1.0], [(1.25, 0.75, 0.75), 0.5]):
        params = ti.Params(p.window, p.falloff, p.strength, p.cap, binding=gains is not None,
                           gains=gains or ())
        mask = None if m == 1.0 else np.full(n, m, np.float32)
        o, lse = oracle.attention_head(q, k, v, lay.seg, _exact_time(lay), lay.picture, mask, params)
        exp = _q0_expected(lay, pen_by_df, gains, m)
        tgt = lay.seg == ti.SEG_TARGET
        for i in np.nonzero(tgt)[0]:
            el, gm, pm = exp[int(lay.frame[i])]
            assert abs(lse[i] - el) < 1e-12
            assert abs(o[i, 0] - gm) < 1e-12
            assert abs(o[i, 1] - pm) < 1e-12
            assert abs(o[i, 2] - 1.0) < 1e-12
        # every other query keeps the plain rule: uniform over all n keys
        assert np.allclose(lse[~tgt], math.log(n), atol=1e-12, rtol=0)
        assert np.allclose(o[~tgt, 0], np.sum(lay.seg == ti.SEG_GUIDE) / n, atol=1e-12, rtol=0)


def test_p4_symmetric_frames():
    lay = ti.make_layout(6, (4, 4), (4, 4), 1, 16, 32)
    n = lay.n
    q = np.zeros((n, 8))
    k = np.ones((n, 8))
    o, lse = oracle.attention_head(q, k, _probe_v(lay), lay.seg, _exact_time(lay), lay.picture, None, DEFAULTS)
    by_frame = {}
    for i in np.nonzero(lay.seg == ti.SEG_TARGET)[0]:
        by_frame.setdefault(int(lay.frame[i]), lse[i])
    for f in range(6):
        assert abs(by_frame[f] - by_frame[5 - f]) < 1e-12


# -------------------------------------------------- P5: weight multiplied by gain^m
def test_p5_gain_power_m_multiplies_unnormalised_weight():
    rng = np.random.default_rng(5)
    lay = ti.make_layout(3, (2, 3), (2, 3), 2, 5, 4, mask=True)
    n = lay.n
    q, k = rng.standard_normal((n, 16)), rng.standard_normal((n, 16))
    eye = np.eye(n)                                   # O row = attention weights
    g = (1.7, 0.6)
    w1, l1 = oracle.attention_head(q, k, eye, lay.seg, lay.time, lay.picture, lay.mask,
                                   ti.Params(binding=True, gains=(1.0, 1.0)))
    wg, lg = oracle.attention_head(q, k, eye, lay.seg, lay.time, lay.picture, lay.mask,
                                   ti.Params(binding=True, gains=g))
    for i in range(n):
        renorm = math.exp(l1[i] - lg[i])
        for j in range(n):
            factor = 1.0
            if lay.seg[i] == ti.SEG_TARGET and lay.seg[j] == ti.SEG_PICTURE:
                factor = g[int(lay.picture[j])] ** float(lay.mask[i])
            assert abs(wg[i, j] - w1[i, j] * factor * renorm) < 1e-13


# ------------------------------------------------------------ P6: brute force
@pytest.mark.parametrize("seed", range(6))
def test_p6_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 25))
    d = int(rng.integers(1, 9))
    lay = ti.random_layout(rng, n, frames=5, pictures=3, mask=bool(seed % 2))
    p = ti.random_params(rng, 3)
    q, k, v = (rng.standard_normal((n, d)) * 1.5 for _ in range(3))
    o, l = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, lay.mask, p)
    bo, bl = oracle.attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), lay.seg, lay.time,
                                         lay.picture, lay.mask, p)
    assert np.max(np.abs(o - bo)) < 1e-12
    assert np.max(np.abs(l - bl)) < 1e-12


# ------------------------------------------------------ P7: partition merge
@pytest.mark.parametrize("seed", range(3))
def test_p7_partition_merge_identity(seed):
    rng = np.random.default_rng(200 + seed)
    lay = ti.random_layout(rng, 150, frames=6, pictures=2)
    p = ti.random_params(rng, 2, binding=True)
    q, k, v = (rng.standard_normal((150, 12)) for _ in range(3))
    full = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, lay.mask, p)
    cuts = np.sort(rng.integers(0, 151, size=int(rng.integers(1, 5))))
    bounds = [0] + [int(c) for c in cuts] + [150]
    parts = [oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, lay.mask, p,
                                   key_range=(a, b)) for a, b in zip(bounds[:-1], bounds[1:])]
    o, l = oracle.merge_partitions(parts)
    assert np.max(np.abs(o - full[0])) < 1e-12
    assert np.max(np.abs(l - full[1])) < 1e-12


# ------------------------------------------------------ P8: three-term identity
def test_p8_three_nonnegative_terms():
    """Target-row normaliser = unbiased keys + all guide keys at -cap + local correction.

    Reading of the article's Flash Partitions backend ("merging three
    non-negative contributions"): sum_k e^z splits exactly into
    sum_unbiased e^s + e^-cap sum_guide e^s + sum_guide e^s (e^-p - e^-cap).
    """
    rng = np.random.default_rng(9)
    lay = ti.make_layout(8, (3, 3), (3, 3), 1, 7, 5)
    n, d = lay.n, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    p = DEFAULTS
    _, lse = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, None, p)
    s = (q @ k.T) / math.sqrt(d)
    guide = lay.seg == ti.SEG_GUIDE
    for i in np.nonzero(lay.seg == ti.SEG_TARGET)[0]:
        dt = np.abs(float(lay.time[i]) - lay.time[guide].astype(np.float64))
        pen = np.array([min(p.strength * (max(x - p.window, 0.0) / p.falloff) ** 2, p.cap) for x in dt])
        t1 = np.exp(s[i, ~guide]).sum()
        t2 = math.exp(-p.cap) * np.exp(s[i, guide]).sum()
        t3 = (np.exp(s[i, guide]) * (np.exp(-pen) - math.exp(-p.cap))).sum()
        assert t1 >= 0 and t2 >= 0 and t3 >= 0
        assert abs(math.log(t1 + t2 + t3) - lse[i]) < 1e-12


@pytest.mark.parametrize("case", ["defaults", "binding", "strength0", "shuffled"])
def test_p8_three_term_parts_merge_to_attention(case):
    """The three terms as LSE partitions (unbiased/binding keys; guide keys at
    -cap; local correction) merge exactly into the full result, row by row,
    and every target row's correction term vanishes past the saturation gap."""
    rng = np.random.default_rng(91)
    lay = ti.make_layout(8, (3, 3), (3, 3), 2, 7, 5, mask=True)
    if case == "shuffled":
        lay = lay.permuted(rng.permutation(lay.n))
    n, d = lay.n, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    p = {"defaults": DEFAULTS, "binding": BIND5, "strength0": ti.Params(strength=0.0),
         "shuffled": BIND5}[case]
    parts = oracle.three_term_parts(q, k, v, lay.seg, lay.time, lay.picture, lay.mask, p)
    o, l = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, lay.mask, p)
    om, lm = oracle.merge_partitions(parts)
    assert np.max(np.abs(om - o)) < 1e-12 and np.max(np.abs(lm - l)) < 1e-12
    tgt = lay.seg == ti.SEG_TARGET
    if case == "strength0":
        assert np.all(np.isneginf(parts[1][1])) and np.all(np.isneginf(parts[2][1]))
        return
    # non-target rows have no correction term; B is the guide keys' plain LSE shifted by -cap on target rows
    assert np.all(np.isneginf(parts[2][1][~tgt]))
    g = lay.seg == ti.SEG_GUIDE
    s = (q @ k.T) / math.sqrt(d)
    plain_b = np.log(np.exp(s[:, g]).sum(axis=1))
    assert np.max(np.abs(parts[1][1] - (plain_b - np.where(tgt, p.cap, 0.0)))) < 1e-12
    # the correction of a target row only sees guide keys closer than the saturation gap
    dsat = tor.saturation_gap(p.window, p.falloff, p.strength, p.cap)
    for i in np.nonzero(tgt)[0]:
        near = g & (np.abs(lay.time.astype(np.float64) - float(lay.time[i])) < dsat)
        pen = tor.penalty(float(lay.time[i]) - lay.time[near].astype(np.float64), p.window, p.falloff,
                          p.strength, p.cap)
        w = np.exp(s[i, near]) * (np.exp(-pen) - math.exp(-p.cap))
        want = math.log(w.sum()) if w.sum() > 0 else -math.inf
        assert abs(parts[2][1][i] - want) < 1e-12 or (want == -math.inf and parts[2][1][i] == -math.inf)


# ----------------------------------------------------------- P9: invariances
def test_p9_invariances():
    rng = np.random.default_rng(21)
    lay = ti.make_layout(5, (3, 4), (3, 4), 2, 6, 7, mask=True)
    n, d = lay.n, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    p = ti.Params(binding=True, gains=(1.4, 0.8))
    o, l = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, lay.mask, p)
    # token permutation with metadata permutes the rows
    perm = rng.permutation(n)
    lp = lay.permuted(perm)
    op, lpp = oracle.attention_head(q[perm], k[perm], v[perm], lp.seg, lp.time, lp.picture, lp.mask, p)
    assert np.max(np.abs(op - o[perm])) < 1e-12 and np.max(np.abs(lpp - l[perm])) < 1e-12
    # a common time shift of every video token changes nothing
    sh = lay.time.astype(np.float64) + 3.25
    os_, ls_ = oracle.attention_head(q, k, v, lay.seg, sh, lay.picture, lay.mask, p)
    assert np.max(np.abs(os_ - o)) < 1e-12 and np.max(np.abs(ls_ - l)) < 1e-12
    # non-target rows ignore the TARA controls
    o2, l2 = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, lay.mask,
                                   ti.Params(0.05, 0.1, 5.0, 9.0, binding=True, gains=(3.0, 0.2)))
    nt = lay.seg != ti.SEG_TARGET
    assert np.array_equal(o2[nt], o[nt]) and np.array_equal(l2[nt], l[nt])
    # heads and batch elements are independent
    q4 = np.stack([q, q * 0.5])[None]
    k4 = np.stack([k, k[::-1]])[None]
    v4 = np.stack([v, v])[None]
    ob, lb = oracle.attention(q4, k4, v4, lay.seg[None], lay.time[None], lay.picture[None],
                              lay.mask[None], p)
    assert np.max(np.abs(ob[0, 0] - o)) < 1e-12 and np.max(np.abs(lb[0, 0] - l)) < 1e-12
    o1, l1 = oracle.attention_head(q * 0.5, k[::-1], v, lay.seg, lay.time, lay.picture, lay.mask, p)
    assert np.max(np.abs(ob[0, 1] - o1)) < 1e-12 and np.max(np.abs(lb[0, 1] - l1)) < 1e-12


def test_p9_batched_attention_matches_bruteforce_per_batch():
    """oracle.attention at B = 2, H = 2, where the two batch elements have
    different metadata and two chained bindings with their own mask planes
    ([J, B, N]): every (b, h) equals the pure-Python brute force run on that
    batch element's own metadata and mask planes. A batch-index slip in the
    metadata or in the mask planes would mix the two layouts and fail."""
    rng = np.random.default_rng(57)
    n, d = 19, 5
    lays = [ti.random_layout(rng, n, frames=4, pictures=2, mask=True) for _ in range(2)]
    for lay in lays:
        assert (lay.seg == ti.SEG_TARGET).any() and (lay.seg == ti.SEG_PICTURE).any()
    assert not np.array_equal(lays[0].seg, lays[1].seg)
    # mask planes [J=2, B=2, N]: each batch element's own first plane and a second random plane
    masks = np.stack([np.stack([lay.mask, rng.uniform(0.0, 1.0, n).astype(np.float32)]) for lay in lays], axis=1)
    p = ti.Params(window=0.1, falloff=0.3, strength=3.0, cap=5.0, binding=True, gains=(1.9, 0.6),
                  chained=((0.7, 2.2),))
    q, k, v = (rng.standard_normal((2, 2, n, d)) for _ in range(3))
    seg = np.stack([x.seg for x in lays])
    tim = np.stack([x.time for x in lays])
    pic = np.stack([x.picture for x in lays])
    ob, lb = oracle.attention(q, k, v, seg, tim, pic, masks, p)
    for b in range(2):
        for h in range(2):
            bo, bl = oracle.attention_bruteforce(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), lays[b].seg,
                                                 lays[b].time, lays[b].picture, masks[:, b], p)
            assert np.max(np.abs(ob[b, h] - bo)) < 1e-12 and np.max(np.abs(lb[b, h] - bl)) < 1e-12
    # the two batch elements really differ (so a swap would be caught)
    o_swapped, _ = oracle.attention(q, k, v, seg[::-1], tim[::-1], pic[::-1], masks[:, ::-1], p)
    assert np.max(np.abs(o_swapped - ob)) > 1e-3


# ----------------------------------------------------------- P10: monotonicity
def test_p10_monotone_guide_mass():
    rng = np.random.default_rng(33)
    lay = ti.make_layout(6, (3, 3), (3, 3), 1, 5, 5)
    n = lay.n
    q, k = rng.standard_normal((n, 16)), rng.standard_normal((n, 16))
    v = _probe_v(lay)
    tgt = lay.seg == ti.SEG_TARGET

    def mass(**kw):
        p = dict(window=0.2, falloff=0.25, strength=2.0, cap=6.0)
        p.update(kw)
        o, _ = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, None, ti.Params(**p))
        return o[tgt, 0]

    for name, vals, sign in (("strength", [0.0, 0.5, 1, 2, 4, 8], -1), ("cap", [0.0, 1, 3, 6, 12], -1),
                             ("window", [0.0, 0.1, 0.2, 0.4, 1.0], 1), ("falloff", [0.05, 0.1, 0.25, 0.5, 2], 1)):
        ms = [mass(**{name: x}) for x in vals]
        for a, b in zip(ms[:-1], ms[1:]):
            assert np.all(sign * (b - a) >= -1e-15), name


# ------------------------------------------------ P11: chained bindings
# "BFS H3 Reference Attention Binding (Experimental)", section "Common issues":
# chained binding nodes add their log gains, so picture i's unnormalised weight
# for a target row is multiplied by prod_j gain_j,i ** m_j.
def _two_plane_mask(lay, rng):
    tgt = lay.seg == ti.SEG_TARGET
    planes = np.zeros((2, lay.n), dtype=np.float32)
    planes[0, tgt] = rng.uniform(0.0, 1.0, int(tgt.sum()))
    planes[1, tgt] = rng.uniform(0.0, 1.0, int(tgt.sum()))
    return planes


def test_p11_equal_masks_multiply_gains():
    rng = np.random.default_rng(11)
    lay = ti.make_layout(4, (3, 3), (3, 3), 3, 6, 5, mask=True)
    q, k, v = (rng.standard_normal((lay.n, 12)) for _ in range(3))
    g1, g2 = (1.6, 0.7, 1.1), (0.5, 1.9, 1.3)
    both = np.stack([lay.mask, lay.mask])
    o2, l2 = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, both,
                                   ti.Params(binding=True, gains=g1, chained=(g2,)))
    o1, l1 = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, lay.mask,
                                   ti.Params(binding=True, gains=tuple(a * b for a, b in zip(g1, g2))))
    assert np.max(np.abs(o2 - o1)) < 1e-12 and np.max(np.abs(l2 - l1)) < 1e-12


def test_p11_neutral_chained_binding_bit_identical():
    rng = np.random.default_rng(12)
    lay = ti.make_layout(4, (3, 3), (3, 3), 2, 6, 5, mask=True)
    q, k, v = (rng.standard_normal((lay.n, 8)) for _ in range(3))
    g = (1.3, 0.8)
    o1, l1 = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, lay.mask,
                                   ti.Params(binding=True, gains=g))
    zero_plane = np.stack([lay.mask, np.zeros_like(lay.mask)])
    for mask, chained in ((np.stack([lay.mask, lay.mask]), ((1.0, 1.0),)),      # gain 1 is neutral
                          (zero_plane, ((2.5, 0.3),))):                          # m = 0 is neutral
        o2, l2 = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, mask,
                                       ti.Params(binding=True, gains=g, chained=chained))
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_p11_q0_closed_form_two_bindings():
    """Q = 0 and no temporal term: every logit is its bias, so per row
    Z = n_other + sum_i n_i * prod_j g_j,i ** m_j,q, LSE = ln Z and the mass on
    picture i is n_i * prod_j g_j,i ** m_j,q / Z (counts from the layout)."""
    rng = np.random.default_rng(13)
    lay = ti.make_layout(3, (2, 3), (2, 3), 3, 5, 4, mask=True)
    planes = _two_plane_mask(lay, rng)
    g = ((1.7, 0.6, 1.2), (0.8, 2.2, 0.9))
    n = lay.n
    q = np.zeros((n, 8))
    k = rng.standard_normal((n, 8))
    v = np.zeros((n, 3))
    for i in range(3):
        v[lay.picture == i, i] = 1.0
    p = ti.Params(strength=0.0, binding=True, gains=g[0], chained=(g[1],))
    o, l = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, planes, p)
    counts = [int(np.sum((lay.seg == ti.SEG_PICTURE) & (lay.picture == i))) for i in range(3)]
    n_other = n - sum(counts)
    for r in range(n):
        if lay.seg[r] == ti.SEG_TARGET:
            w = [counts[i] * (g[0][i] ** float(planes[0, r])) * (g[1][i] ** float(planes[1, r])) for i in range(3)]
        else:
            w = [float(c) for c in counts]
        z = n_other + sum(w)
        assert abs(l[r] - math.log(z)) < 1e-13
        for i in range(3):
            assert abs(o[r, i] - w[i] / z) < 1e-13


def test_p11_binding_order_and_bruteforce():
    rng = np.random.default_rng(14)
    for trial in range(4):
        n = int(rng.integers(4, 20))
        lay = ti.random_layout(rng, n, frames=4, pictures=3, mask=True)
        planes = _two_plane_mask(lay, rng)
        p = ti.random_params(rng, 3, binding=True)
        g2 = tuple(float(x) for x in rng.uniform(0.3, 2.5, size=3))
        q, k, v = (rng.standard_normal((n, 5)) for _ in range(3))
        pa = ti.Params(p.window, p.falloff, p.strength, p.cap, True, p.gains, (g2,))
        pb = ti.Params(p.window, p.falloff, p.strength, p.cap, True, g2, (tuple(p.gains),))
        oa, la = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, planes, pa)
        ob, lb = oracle.attention_head(q, k, v, lay.seg, lay.time, lay.picture, planes[::-1].copy(), pb)
        assert np.max(np.abs(oa - ob)) < 1e-13 and np.max(np.abs(la - lb)) < 1e-13
        bo, bl = oracle.attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), lay.seg, lay.time,
                                             lay.picture, planes, pa)
        assert np.max(np.abs(oa - bo)) < 1e-12 and np.max(np.abs(la - bl)) < 1e-12


# ---------------------------------------------------- P12: 8-bit Q.K scheme
def test_p12_fp8_e4m3_hand_worked(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "fp8_e4m3_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                a, b = line.split()
                rows.append((float(a), float(b)))
    assert len(rows) >= 12
    got = oracle.fp8_e4m3_round(np.array([r[0] for r in rows]))
    assert np.array_equal(got, np.array([r[1] for r in rows]))


def test_p12_fp8_e4m3_against_code_table():
    """Every E4M3 code's value rounds to itself; points between two adjacent
    values round to the nearer one, midpoints to the one with an even code."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                                     # NaN code
            vals.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    vals = np.array(sorted(set(vals)))                       # 0 .. 448, codes in increasing order
    assert vals[-1] == 448.0 and len(vals) == 127
    assert np.array_equal(oracle.fp8_e4m3_round(vals), vals)
    assert np.array_equal(oracle.fp8_e4m3_round(-vals), -vals)
    lo, hi = vals[:-1], vals[1:]
    mid = (lo + hi) / 2
    codes = np.arange(len(vals))
    even_pick = np.where(codes[:-1] % 2 == 0, lo, hi)
    assert np.array_equal(oracle.fp8_e4m3_round(mid), even_pick)
    assert np.array_equal(oracle.fp8_e4m3_round(lo + (hi - lo) * 0.3), lo)
    assert np.array_equal(oracle.fp8_e4m3_round(lo + (hi - lo) * 0.7), hi)


def test_p12_scales_and_dequantised_error():
    rng = np.random.default_rng(120)
    q = rng.standard_normal((300, 64)) * np.exp(rng.uniform(-6, 6, size=(300, 1)))
    # key tiles of 64 rows with magnitudes apart by up to e^8
    k = rng.standard_normal((300, 64)) * 3.0 * np.repeat(np.exp(rng.uniform(-4, 4, size=(5, 1))), 64, axis=0)[:300]
    for row in q[:20]:
        s = oracle.pow2_scale(float(np.abs(row).max()))
        assert math.log2(s) == int(math.log2(s)) and 128.0 <= np.abs(row).max() / s < 256.0
    assert oracle.pow2_scale(0.0) == 1.0
    qd, kd = oracle.qk8_dequantize(q, k)
    for x, xd, tile in ((q, qd, 1), (k, kd, 64)):
        for t0 in range(0, x.shape[0], tile):
            blk, bd = x[t0:t0 + tile], xd[t0:t0 + tile]
            s = oracle.pow2_scale(float(np.abs(blk).max()))
            normal = np.abs(blk) / s >= 2.0 ** -6
            # half an ulp: 2^-4 relative for normals, 2^-10 * scale below
            assert np.all(np.abs(bd - blk)[normal] <= np.abs(blk)[normal] * 2.0 ** -4)
            assert np.all(np.abs(bd - blk)[~normal] <= s * 2.0 ** -10)
            # the largest element of every row / tile is a normal E4M3 value in [128, 256) * s
            assert 128.0 <= np.abs(bd).max() / s <= 256.0


# ----------------------------------------------------- planted mistakes fail a pin
def _pins_pass(golden_dir):
    fx = _load_penalty_fixture(golden_dir)
    checks = [lambda: test_p1_penalty_closed_form(fx),
              lambda: test_p2_reduces_to_sdpa("strength0"),
              lambda: test_p4_q0_closed_form(fx, "defaults"),
              lambda: test_p4_q0_closed_form(fx, "binding"),
              lambda: test_p5_gain_power_m_multiplies_unnormalised_weight(),
              lambda: test_p6_bruteforce(1),
              lambda: test_p7_partition_merge_identity(0),
              lambda: test_p11_q0_closed_form_two_bindings(),
              lambda: test_p8_three_term_parts_merge_to_attention("defaults"),
              lambda: test_p12_fp8_e4m3_hand_worked(golden_dir),
              lambda: test_p12_fp8_e4m3_against_code_table(),
              lambda: test_p12_scales_and_dequantised_error(),
              lambda: test_p9_batched_attention_matches_bruteforce_per_batch()]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def test_pins_catch_planted_mistakes(golden_dir, monkeypatch):
    assert _pins_pass(golden_dir)
    real_pen, real_bias, real_head = tor.penalty, tor.bias_block, tor.attention_head

    def no_square(dt, w, f, s, c):
        x = np.maximum(np.abs(np.asarray(dt, np.float64)) - w, 0.0) / f
        return np.minimum(s * x, c)

    def no_window(dt, w, f, s, c):
        return real_pen(dt, 0.0, f, s, c)

    def wrong_sign(*a, **kw):
        return -real_bias(*a, **kw)

    def swap_qk_roles(seg_q, tq, mq, seg_k, tk, pk, params):
        # bias the guide-query x target-key edges instead
        sq = np.where(seg_q == tor.GUIDE, tor.TARGET, np.where(seg_q == tor.TARGET, tor.GUIDE, seg_q))
        sk = np.where(seg_k == tor.GUIDE, tor.TARGET, np.where(seg_k == tor.TARGET, tor.GUIDE, seg_k))
        return real_bias(sq, tq, mq, sk, tk, pk, params)

    def log2_gain(seg_q, tq, mq, seg_k, tk, pk, params):
        b = real_bias(seg_q, tq, mq, seg_k, tk, pk, params)
        return b / math.log(2.0) if params.binding else b

    def transposed_kv(q, k, v, *a, **kw):
        return real_head(q, v, k, *a, **kw) if q.shape == v.shape else real_head(q, k, v, *a, **kw)

    def first_binding_only(seg_q, tq, mq, seg_k, tk, pk, params):
        # chained bindings dropped, the first mask plane kept
        first = ti.Params(params.window, params.falloff, params.strength, params.cap, params.binding,
                          params.gains)
        planes = None if mq is None else np.asarray(mq).reshape(getattr(params, "num_bindings", 1), -1)
        return real_bias(seg_q, tq, None if planes is None else planes[0], seg_k, tk, pk, first)

    def one_mask_plane(seg_q, tq, mq, seg_k, tk, pk, params):
        # every binding weighted by the first binding's mask
        nb = getattr(params, "num_bindings", 1)
        if mq is None or nb == 1:
            return real_bias(seg_q, tq, mq, seg_k, tk, pk, params)
        planes = np.asarray(mq).reshape(nb, -1)
        return real_bias(seg_q, tq, np.stack([planes[0]] * nb), seg_k, tk, pk, params)

    real_three = tor.three_term_parts

    def correction_keeps_cap(*a, **kw):
        # local correction without subtracting the cap contribution (counts it twice)
        parts = real_three(*a, **kw)
        q, k, v, seg, time, picture, mask, params = a[:8]
        s = np.asarray(q, np.float64) @ np.asarray(k, np.float64).T / math.sqrt(np.asarray(q).shape[1])
        g = np.asarray(seg) == tor.GUIDE
        tgt = np.asarray(seg) == tor.TARGET
        pen = np.zeros_like(s)
        tm = np.asarray(time, np.float64)
        pen[:, g] = tor.penalty(tm[:, None] - tm[g][None, :], params.window, params.falloff, params.strength,
                                params.cap)
        zc = np.where(g[None, :] & tgt[:, None], s - pen, -np.inf)
        l = np.full(s.shape[0], -np.inf)
        ok = tgt & g.any()
        l[ok] = np.log(np.exp(zc[ok]).sum(axis=1))
        return [parts[0], parts[1], (parts[2][0], l)]

    def fp8_truncating(x):
        # rounding toward zero instead of to nearest even
        x = np.asarray(x, np.float64)
        a = np.abs(x)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        ulp = 2.0 ** (np.maximum(e, -6.0) - 3.0)
        return np.sign(x) * np.floor(a / ulp) * ulp

    def fp8_half_away(x):
        # ties away from zero instead of to even
        x = np.asarray(x, np.float64)
        a = np.abs(x)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        ulp = 2.0 ** (np.maximum(e, -6.0) - 3.0)
        return np.sign(x) * np.floor(a / ulp + 0.5) * ulp

    real_scale, real_deq = tor.pow2_scale, tor.qk8_dequantize

    def scale_one_low(amax):
        # largest magnitude lands in [64, 128): one bit of precision lost
        return real_scale(amax) * 2.0

    def per_tensor_k_scale(q, k, tile=64):
        # one scale for all of K instead of one per key tile
        return real_deq(q, k, tile=max(1, np.asarray(k).shape[0]))

    def no_cap(dt, w, f, s, c):
        # the quadratic never saturates
        x = np.maximum(np.abs(np.asarray(dt, np.float64)) - w, 0.0) / f
        return s * x * x

    def guide_rows_biased_too(seg_q, tq, mq, seg_k, tk, pk, params):
        # guide queries treated like target queries
        return real_bias(np.where(np.asarray(seg_q) == tor.GUIDE, tor.TARGET, seg_q), tq, mq, seg_k, tk, pk, params)

    def binding_on_every_row(seg_q, tq, mq, seg_k, tk, pk, params):
        # the binding term added for every query row, not only target rows
        b = real_bias(seg_q, tq, mq, seg_k, tk, pk, params)
        if not params.binding:
            return b
        seg_q = np.asarray(seg_q)
        other = seg_q != tor.TARGET
        if not other.any():
            return b
        only_binding = ti.Params(params.window, params.falloff, 0.0, params.cap, params.binding, params.gains,
                                 chained=params.chained)
        nb = getattr(params, "num_bindings", 1)
        ones = None if mq is None else np.ones((nb, seg_q.shape[0]))
        ball = real_bias(np.full_like(seg_q, tor.TARGET), tq, ones, seg_k, tk, pk, only_binding)
        return b + np.where(other[:, None], ball, 0.0)

    def bias_scaled_like_logits(*a, **kw):
        # the bias multiplied by the softmax scale of a 64-wide head
        return real_bias(*a, **kw) * 0.125

    def mask_ignored(seg_q, tq, mq, seg_k, tk, pk, params):
        # m = 1 on every target query whatever the mask says
        return real_bias(seg_q, tq, None, seg_k, tk, pk, params)

    real_attention = tor.attention

    def batch0_metadata(q, k, v, seg, time, picture, mask, params, **kw):
        # every batch element reads batch element 0's metadata and mask planes
        seg, time, picture = (np.repeat(np.asarray(x)[:1], np.asarray(x).shape[0], axis=0)
                              for x in (seg, time, picture))
        if mask is not None:
            mk = np.asarray(mask)
            mask = np.repeat(mk[..., :1, :], mk.shape[-2], axis=-2)
        return real_attention(q, k, v, seg, time, picture, mask, params, **kw)

    mutants = [("pow2_scale", scale_one_low), ("qk8_dequantize", per_tensor_k_scale),
               ("penalty", no_cap), ("bias_block", guide_rows_biased_too), ("bias_block", binding_on_every_row),
               ("bias_block", bias_scaled_like_logits), ("bias_block", mask_ignored),
               ("penalty", no_square), ("penalty", no_window), ("bias_block", wrong_sign),
               ("bias_block", swap_qk_roles), ("bias_block", log2_gain), ("attention_head", transposed_kv),
               ("bias_block", first_binding_only), ("bias_block", one_mask_plane),
               ("three_term_parts", correction_keeps_cap), ("fp8_e4m3_round", fp8_truncating),
               ("fp8_e4m3_round", fp8_half_away), ("attention", batch0_metadata)]
    for name, fn in mutants:
        with monkeypatch.context() as m:
            m.setattr(tor, name, fn)
            if name in ("attention_head", "three_term_parts", "fp8_e4m3_round", "pow2_scale", "qk8_dequantize",
                        "attention"):
                m.setattr(oracle, name, fn)
            assert not _pins_pass(golden_dir), f"planted mistake {fn.__name__} went unnoticed"
