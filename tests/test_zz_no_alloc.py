"""tara_attn_fwd_noalloc against tara_attn_fwd, through the C ABI.

The allocation-free entry point runs the same kernels on its own fixed device
array, one batch element and as many heads as the array holds at a time, so
its outputs must equal the workspace entry point's exactly. Two calls in a
row, the second smaller: the benchmark's 107,126-token sequence at 9 heads
(three groups of heads through the array), then a small two-element batch
with two chained bindings (each batch element reads its own rows of both mask
planes). A fused call with a tail split run in groups of heads. Then the
partitioned and three-term modes, and the rejection of a call whose single
head needs more than the array holds.
"""
import numpy as np
import pytest
import torch

import tara_inputs as ti
import temporally_biased_flashattention_amd as tara
from tara_testlib import device_meta, log, tara_params

pytestmark = pytest.mark.gpu

CHAIN = ti.Params(window=0.10, falloff=0.40, strength=3.0, cap=8.0, binding=True, gains=(1.25, 0.75, 0.75),
                  chained=((0.8, 1.4, 1.1),))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(q, k, v, lay, p, B, mode="fused", partitions=1, bounds=None, mask=None):
    """(O, LSE) of tara_attn_fwd and of tara_attn_fwd_noalloc on the same
    inputs (mask: a device mask tensor to use instead of the layout's)."""
    seg, tim, pic, lay_mask = device_meta(lay, "cuda", B)
    mask = lay_mask if mask is None else mask
    params = tara_params(p, mode, partitions, bounds)
    o1, l1 = tara.attn_fwd(q, k, v, seg, tim, pic, mask, params)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    tara.tara_attn_fwd_noalloc(q, k, v, o2, l2, seg, tim, pic, mask, params)
    info = tara.tara_get_last_run_info()
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2), info


def _same(a, b, what):
    (o1, l1), (o2, l2) = a, b
    do = float((o1.float() - o2.float()).abs().max())
    dl = float((l1 - l2).abs().max())
    log(f"{what}: no-alloc vs workspace entry point: max|dO|={do:.3e} max|dLSE|={dl:.3e}")
    assert bool(torch.isfinite(o2).all()) and bool(torch.isfinite(l2).all())
    assert torch.equal(o1, o2) and torch.equal(l1, l2), what


def test_noalloc_matches_two_calls_second_smaller():
    # first call: 107,126 tokens x 9 heads x d128 (the array holds 4 heads' workspace at this length)
    lay = ti.config(6).layout()
    g = torch.Generator().manual_seed(5100)
    q, k, v = (torch.randn(1, 9, lay.n, 128, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    a, b, info = _both(q, k, v, lay, ti.Params(), 1)
    assert info["grid"] == 419 * 9, info
    _same(a, b, "107,126 tokens x 9 heads")
    del q, k, v, a, b
    # second call, smaller: B = 2, 3 heads, d64, two chained bindings with their own mask planes
    lay2 = ti.make_layout(12, (8, 16), (8, 16), 3, 100, 50, mask=True)
    rng = np.random.default_rng(5101)
    lay2 = ti.Layout(lay2.seg, lay2.time, lay2.picture, lay2.frame,
                     np.stack([lay2.mask, (rng.uniform(0, 1, lay2.n) * (lay2.seg == 0)).astype(np.float32)]))
    g = torch.Generator().manual_seed(5102)
    q, k, v = (torch.randn(2, 3, lay2.n, 64, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    # BNHD views: strided heads
    q, k, v = (x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for x in (q, k, v))
    # mask planes [2 bindings, 2 batch elements, N], different for every (binding, batch element)
    tgt = torch.from_numpy(lay2.seg == 0).float()
    mask = (torch.rand(2, 2, lay2.n, generator=g) * tgt).cuda()
    _same(*_both(q, k, v, lay2, CHAIN, 2, mask=mask)[:2], f"B=2 x 3 heads x {lay2.n} tokens, chained bindings")


def test_noalloc_tail_split_in_groups():
    """107,126 tokens x 8 heads x d128: the fused call hands each head's last
    630 rows to the range pass over ten key ranges (its workgroups would leave
    the last round of compute units nearly empty). The call needs more than the
    array, so the no-alloc entry point runs it in groups of heads; every group
    keeps the call's split, and the outputs equal the workspace entry point's."""
    lay = ti.config(6).layout()
    g = torch.Generator().manual_seed(5105)
    q, k, v = (torch.randn(1, 8, lay.n, 128, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    a, b, info = _both(q, k, v, lay, ti.Params(), 1)
    log(f"no-alloc run info: {info}")
    assert info["grid"] == 8 * 416 + 8 * 3 * 10, info
    _same(a, b, "107,126 tokens x 8 heads, tail split")


@pytest.mark.parametrize("mode", ["partitioned", "three-term", "frame-loop"])
def test_noalloc_other_modes(mode):
    lay = ti.make_layout(12, (8, 16), (8, 16), 3, 100, 50, mask=True)
    g = torch.Generator().manual_seed(5103)
    q, k, v = (torch.randn(2, 5, lay.n, 128, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    p = ti.Params(window=0.10, falloff=0.40, strength=3.0, cap=8.0, binding=True, gains=(1.25, 0.75, 0.75))
    bounds = {"partitioned": [0, 100, 777, lay.n], "frame-loop": ti.frame_loop_bounds(lay)}.get(mode)
    parts = len(bounds) - 1 if bounds else 1
    _same(*_both(q, k, v, lay, p, 2, mode, parts, bounds)[:2], f"{mode}, B=2 x 5 heads")


def test_noalloc_fp32_and_qk8():
    lay = ti.make_layout(6, (6, 10), (6, 10), 2, 40, 37, mask=True)
    g = torch.Generator().manual_seed(5104)
    q, k, v = (torch.randn(1, 2, lay.n, 64, generator=g).cuda() for _ in range(3))
    _same(*_both(q, k, v, lay, ti.Params(), 1)[:2], "fp32")
    seg, tim, pic, mask = device_meta(lay, "cuda", 1)
    qb, kb, vb = (x.to(torch.bfloat16) for x in (q, k, v))
    params = tara.make_params(qk8=True)
    o1, l1 = tara.attn_fwd(qb, kb, vb, seg, tim, pic, mask, params)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    tara.tara_attn_fwd_noalloc(qb, kb, vb, o2, l2, seg, tim, pic, mask, params)
    torch.cuda.synchronize()
    _same((o1, l1), (o2, l2), "8-bit Q.K")


def test_noalloc_rejects_a_head_beyond_the_array():
    """The dense-bias baseline's bias tensor alone is N * npad * 4 bytes: at
    N = 8,192 that is 256 MiB, beyond the 128 MiB array."""
    n = 8192
    lay = ti.make_layout(8, (8, 16), (8, 16), 1, 100, n - 8 * 8 * 16 * 2 - 100)
    assert lay.n == n
    q = torch.zeros(1, 1, n, 64, dtype=torch.bfloat16, device="cuda")
    seg, tim, pic, mask = device_meta(lay, "cuda", 1)
    o, l = torch.empty_like(q), torch.empty(1, 1, n, device="cuda")
    with pytest.raises(tara.TaraError) as e:
        tara.tara_attn_fwd_noalloc(q, q, q, o, l, seg, tim, pic, None, tara.make_params(mode="dense-bias"))
    log(f"rejected: {e.value}")
    assert e.value.status == -7 and "no-alloc" in e.value.detail
