"""The bias tile classes against the per-element formula, through the C ABI.

The bf16 kernel applies the bias of a 64-key tile as one constant per query
row when the tile allows it (plain, saturated past window + falloff *
sqrt(cap/strength), inside the free window, one bound picture) and evaluates
the rule per element otherwise. TARA_DISABLE_TILE_SKIP=1 sends every tile down
the per-element path. Both must give the same attention: at full size, one
fused call over all heads each way, compared element by element over every
output, and each against the fp64 oracle on stratified rows of three heads.
The tile-class counts of the debug readback (TARA_TILE_STATS=1) cover every
(row, key tile) pair once.

Gates between the two GPU results: both paths compute the same fp32 logits
and take the same exponent reference (the row max is updated by the same
threshold rule), so they differ only by the rounding of the bias term: about
one fp32 ulp of a logit, and through it an occasional different bf16 rounding
of a single weight. |dO| <= 1e-3 and |dLSE| <= 1e-5 leave room for that.
"""
import numpy as np
import pytest
import torch

import tara_inputs as ti
import temporally_biased_flashattention_amd as tara
from tara_testlib import compare, device_meta, log, run_oracle, sample_rows, tara_params

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _call(qd, kd, vd, lay, p, monkeypatch, elem_all, mode="fused", partitions=1, bounds=None):
    seg, tim, pic, mask = device_meta(lay, "cuda", 1)
    params = tara_params(p, mode, partitions, bounds)
    with monkeypatch.context() as m:
        m.setenv("TARA_TILE_STATS", "1")
        if elem_all:
            m.setenv("TARA_DISABLE_TILE_SKIP", "1")
        else:
            m.delenv("TARA_DISABLE_TILE_SKIP", raising=False)
        o = torch.full_like(qd, float("nan"))
        lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device=qd.device)
        tara.attn_fwd(qd, kd, vd, seg, tim, pic, mask, params, out=o, lse=lse)
        info = tara.tara_get_last_run_info()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    return o, lse, info


def _key_tiles(n, bounds):
    return sum((b1 + 63) // 64 - b0 // 64 for b0, b1 in zip(bounds[:-1], bounds[1:]) if b1 > b0)


def _check_counts(info, H, n, bounds, elem_all):
    counts = {c: info[f"tiles_{c}"] for c in ("plain", "saturated", "window", "picture", "elem")}
    total = sum(counts.values())
    log(f"tile classes ({'forced per-element' if elem_all else 'classed'}): "
        + ", ".join(f"{c} {v} ({100 * v / total:.2f}%)" for c, v in counts.items()))
    assert info["tile_stats"] == 1 and info["elem_all"] == int(elem_all)
    assert all(v >= 0 for v in counts.values())
    assert total == H * n * _key_tiles(n, bounds)
    if elem_all:
        assert counts["elem"] == total
    return counts


@pytest.mark.parametrize("cid", [5, 6])
def test_tile_classes_match_per_element_fullsize(cid, monkeypatch):
    cfg = ti.config(cid)
    lay = cfg.layout()
    log(f"config {cid} {cfg.name}: N={lay.n} H={cfg.heads}; generating inputs")
    q, k, v = ti.qkv(cfg)
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    oc, lc, ic = _call(qd, kd, vd, lay, cfg.params, monkeypatch, elem_all=False)
    counts = _check_counts(ic, cfg.heads, lay.n, [0, lay.n], False)
    # the constant classes do the work: most pairs take no per-element math
    assert counts["elem"] < 0.1 * sum(counts.values())
    assert counts["saturated"] > 0 and counts["plain"] > 0
    oe, le, ie = _call(qd, kd, vd, lay, cfg.params, monkeypatch, elem_all=True)
    _check_counts(ie, cfg.heads, lay.n, [0, lay.n], True)
    do = float((oc.float() - oe.float()).abs().max())
    dl = float((lc - le).abs().max())
    log(f"config {cid}: classed vs per-element on every output: max|dO|={do:.3e} max|dLSE|={dl:.3e}")
    assert do <= 1e-3 and dl <= 1e-5
    heads = [0, cfg.heads // 2, cfg.heads - 1]
    rows = sample_rows(lay, n_random=128, per_segment=32, seed=700 + cid)
    hi = torch.tensor(heads, device="cuda")
    ri = torch.as_tensor(rows, device="cuda")
    ro, rl = run_oracle(q, k, v, lay, cfg.params, rows=rows, heads=heads)
    for name, o, l in (("classed", oc, lc), ("per-element", oe, le)):
        og = o.index_select(1, hi).index_select(2, ri).float().cpu().numpy()
        lg = l.index_select(1, hi).index_select(2, ri).cpu().numpy()
        compare(og, lg, ro, rl, what=f"config {cid} {name} vs oracle")


def test_tile_classes_partitioned_counts(monkeypatch):
    """Partitioned mode counts the key tiles of every range (a tile that two
    ranges share is visited by both) and agrees with the per-element path."""
    lay = ti.make_layout(12, (8, 16), (8, 16), 3, 100, 50, mask=True)
    p = ti.Params(window=0.10, falloff=0.40, strength=3.0, cap=8.0, binding=True, gains=(1.25, 0.75, 0.75))
    g = torch.Generator().manual_seed(71)
    q, k, v = (torch.randn(1, 2, lay.n, 128, generator=g).to(torch.bfloat16) for _ in range(3))
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    bounds = [0, 100, 777, 1000, lay.n]
    oc, lc, ic = _call(qd, kd, vd, lay, p, monkeypatch, False, "partitioned", 4, bounds)
    _check_counts(ic, 2, lay.n, bounds, False)
    oe, le, ie = _call(qd, kd, vd, lay, p, monkeypatch, True, "partitioned", 4, bounds)
    _check_counts(ie, 2, lay.n, bounds, True)
    assert float((oc.float() - oe.float()).abs().max()) <= 1e-3 and float((lc - le).abs().max()) <= 1e-5
    ro, rl = run_oracle(q, k, v, lay, p)
    compare(oc.float().cpu().numpy(), lc.cpu().numpy(), ro, rl, what="partitioned classed vs oracle")
