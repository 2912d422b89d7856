"""GPU parity of the 8-bit Q.K mode (the dense 8-bit one-pass kernels of the
"Three backends" section; the pages give no quantisation scheme, so the
scheme is the oracle's qk8_dequantize: FP8 E4M3, round to nearest even, a
power-of-two scale per query row and per 64-key tile).

Two gates:
- against the fp64 oracle run on the dequantised Q and K (what the FP8
  products compute exactly, up to fp32 summation): the usual bf16 gates,
  max|dO| <= 1e-2, max|dLSE| <= 1e-3, relative 1e-2;
- against the oracle on the unrounded Q and K, the looser tolerance the
  rounding itself allows. With D_i = max_j |s'_ij - s_ij| the largest change
  of a row's logits (natural-log units; the bias is the same on both sides),
  log-sum-exp is 1-Lipschitz in the max norm, so |dLSE_i| <= D_i; each
  normalised weight moves by a factor within e^(+-2 D_i), so
  |dO_i| <= (e^(2 D_i) - 1) max|V|. Both are added to the bf16 gates.
"""
import numpy as np
import pytest
import torch

import tara_inputs as ti
from tara_testlib import compare, dequantized, log, qkv_random, rounding_gate, run_gpu, run_oracle, sample_rows

pytestmark = pytest.mark.gpu

BIND = ti.Params(window=0.10, falloff=0.40, strength=3.0, cap=8.0, binding=True, gains=(1.25, 0.75, 0.75))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def logit_shift(q, k, qd, kd, scale, heads, rows):
    """D_i = max_j |scale (q'_i . k'_j - q_i . k_j)| per [B, Hs, R], in fp64."""
    out = np.zeros((q.shape[0], len(heads), len(rows)))
    for b in range(q.shape[0]):
        for i, h in enumerate(heads):
            s0 = q[b, h, rows].double() @ k[b, h].double().T
            s1 = qd[b, h, rows].double() @ kd[b, h].double().T
            out[b, i] = (scale * (s1 - s0).abs().max(dim=1).values).numpy()
    return out


def check_qk8(q, k, v, lay, p, what, heads=None, rows=None):
    B, H, N, D = q.shape
    hs = list(range(H)) if heads is None else list(heads)
    rs = np.arange(N) if rows is None else np.asarray(rows)
    o, l = run_gpu(q, k, v, lay, p, qk8=True, heads=heads, rows=rows)
    qd, kd = dequantized(q, k, heads=hs, rows=None if rows is None else rs)
    ro, rl = run_oracle(qd, kd, v, lay, p, rows=rows, heads=hs)
    compare(o.numpy(), l.numpy(), ro, rl, what=f"{what} vs oracle on 8-bit Q,K")
    # against unrounded Q.K: the bound the rounding allows, per row
    xo, xl = run_oracle(q, k, v, lay, p, rows=rows, heads=hs)
    shift = logit_shift(q, k, qd, kd, 1.0 / np.sqrt(D), hs, rs)
    vmax = float(v.float().abs().max())
    dl = np.abs(l.numpy() - xl)
    do = np.abs(o.numpy() - xo).max(axis=-1)
    log(f"{what} vs unrounded: max|dO|={do.max():.3e} max|dLSE|={dl.max():.3e} max row shift={shift.max():.3e}")
    assert (dl <= shift + 1e-3).all(), "LSE moved more than the largest logit shift"
    assert (do <= np.expm1(2.0 * shift) * vmax + 1e-2).all(), "O moved more than the logit shift allows"


@pytest.mark.parametrize("d", [128, 64])
def test_qk8_small(d):
    lay = ti.make_layout(6, (6, 10), (6, 10), 2, 40, 37)
    q, k, v = qkv_random(1, 2, lay.n, d, seed=80 + d)
    check_qk8(q, k, v, lay, ti.Params(), f"qk8 defaults d={d}")


def test_qk8_binding_framed_shuffled():
    lay = ti.make_layout(12, (8, 16), (8, 16), 3, 100, 50, mask=True)
    q, k, v = qkv_random(1, 2, lay.n, 128, seed=83)
    check_qk8(q, k, v, lay, BIND, "qk8 framed binding")
    sh = lay.permuted(np.random.default_rng(84).permutation(lay.n))
    check_qk8(q, k, v, sh, BIND, "qk8 shuffled binding")


def test_qk8_wide_range_scales():
    """Rows and key tiles whose magnitudes differ by powers of two: every Q row
    and K tile gets its own scale; peaky scores (q, k ~ N(0, 4) after the
    scaling). O gate as for the peaky bf16 case (rounding_gate)."""
    lay = ti.make_layout(6, (6, 10), (6, 10), 2, 40, 37, mask=True)
    q, k, v = qkv_random(1, 2, lay.n, 128, seed=85, scale=2.0)
    g = torch.Generator().manual_seed(86)
    rq = torch.exp2(torch.randint(-6, 4, (1, 2, lay.n, 1), generator=g).float())
    rk = torch.exp2(torch.randint(-6, 4, (1, 2, (lay.n + 63) // 64, 1), generator=g).float())
    rk = rk.repeat_interleave(64, dim=2)[:, :, :lay.n]
    q = (q.float() * rq.clamp(max=1.0)).to(torch.bfloat16)
    k = (k.float() * rk.clamp(max=1.0)).to(torch.bfloat16)
    o, l = run_gpu(q, k, v, lay, BIND, qk8=True)
    qd, kd = dequantized(q, k)
    ro, rl = run_oracle(qd, kd, v, lay, BIND)
    compare(o.numpy(), l.numpy(), ro, rl, tol_o=rounding_gate(qd, kd, v, lay, BIND, ro),
            what="qk8 per-row / per-tile magnitudes")


def test_qk8_zero_rows_and_ragged_tail():
    """All-zero Q rows and an all-zero K tile (scale 1, codes 0); N = 285, so
    the last key tile holds 29 keys."""
    lay = ti.make_layout(2, (6, 10), (6, 10), 1, 40, 5)
    assert lay.n % 64 != 0
    q, k, v = qkv_random(1, 2, lay.n, 128, seed=87)
    q[:, :, ::7] = 0
    k[:, :, 64:128] = 0
    check_qk8(q, k, v, lay, ti.Params(), "qk8 zero rows / tile, ragged")


@pytest.mark.parametrize("cid", [2, 5, 6])
def test_qk8_fullsize_sampled(cid):
    """One fused 8-bit call over all heads at full size: workload 2 (54,272
    tokens x 8 heads), the binding workload 5 (107,682 tokens x 56 heads,
    three pictures, a soft mask) and the benchmark workload 6 (107,126 tokens
    x 56 heads, D 128); stratified rows of three heads."""
    cfg = ti.config(cid)
    lay = cfg.layout()
    log(f"config {cid} {cfg.name}: N={lay.n} H={cfg.heads}; generating inputs")
    q, k, v = ti.qkv(cfg)
    heads = [0, cfg.heads // 2, cfg.heads - 1]
    rows = sample_rows(lay, n_random=128, per_segment=32, seed=88 + cid)
    check_qk8(q, k, v, lay, cfg.params, f"qk8 config {cid} sampled", heads=heads, rows=rows)


def test_qk8_rejected_outside_fused_bf16():
    lay = ti.make_layout(2, (6, 10), (6, 10), 1, 40, 5)
    q, k, v = qkv_random(1, 1, lay.n, 64, seed=89)
    import temporally_biased_flashattention_amd as tara
    with pytest.raises(tara.TaraError):
        run_gpu(q, k, v, lay, ti.Params(), qk8=True, mode="three-term")
    qf, kf, vf = (x.float() for x in (q, k, v))
    with pytest.raises(tara.TaraError):
        run_gpu(qf, kf, vf, lay, ti.Params(), qk8=True)
