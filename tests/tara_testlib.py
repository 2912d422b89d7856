"""Helpers shared by the GPU parity tests: run the HIP library and the fp64
oracle on the same seeded inputs and compare them.

The library is reached only through the Python binding of the C ABI; the
oracle only through oracle/. Neither side sees the other's code or results.
"""
from __future__ import annotations

import math
import sys
import time
from typing import Optional, Sequence

import numpy as np
import torch

import oracle
import tara_inputs as ti
import temporally_biased_flashattention_amd as tara
from tara_inputs import sample_rows  # noqa: F401 (re-exported for the tests)

# Gates (max |dO| <= 1e-2 for bf16 inputs with fp32 accumulation, |dLSE| <= 1e-3).
TOL_O = 1e-2
TOL_LSE = 1e-3
TOL_REL_O = 1e-2


def log(msg: str):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def tara_params(p: ti.Params, mode="fused", partitions=1, bounds=None, softmax_scale=0.0, qk8=False):
    return tara.make_params(window=p.window, falloff=p.falloff, strength=p.strength, cap=p.cap,
                            binding=p.binding, gains=tuple(p.gains), softmax_scale=softmax_scale,
                            mode=mode, partitions=partitions, bounds=bounds,
                            chained=tuple(tuple(c) for c in p.chained), qk8=qk8)


def device_meta(lay: ti.Layout, device="cuda", batch=1):
    """Metadata tensors [batch, N] on the device (the same layout per batch
    element); a mask with one plane per binding becomes [J, batch, N]."""
    def rep(x, dt):
        t = torch.from_numpy(np.ascontiguousarray(x)).to(dt)
        return t.unsqueeze(-2).repeat(*([1] * (t.dim() - 1)), batch, 1).contiguous().to(device)
    seg = rep(lay.seg, torch.uint8)
    tim = rep(lay.time, torch.float32)
    pic = rep(lay.picture, torch.int16)
    mask = None if lay.mask is None else rep(lay.mask, torch.float32)
    return seg, tim, pic, mask


def run_gpu(q, k, v, lay: ti.Layout, p: ti.Params, mode="fused", partitions=1, bounds=None,
            softmax_scale=0.0, layout="bhnd", use_mask=True, heads=None, rows=None, qk8=False, poison=False):
    """q, k, v: CPU tensors [B, H, N, D]. Returns (O fp32 CPU, LSE fp32 CPU),
    restricted to the given heads and query rows when those are given.
    poison: O and LSE are filled with NaN before the call, and every element
    of both (all heads and rows) must be finite after it: the call wrote them
    all."""
    dev = "cuda"
    B, H, N, _ = q.shape
    if layout == "bhnd":
        qd, kd, vd = (x.to(dev).contiguous() for x in (q, k, v))
    else:   # stored [B, N, H, D], passed as a [B, H, N, D] view
        qd, kd, vd = (x.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3) for x in (q, k, v))
    seg, tim, pic, mask = device_meta(lay, dev, B)
    params = tara_params(p, mode, partitions, bounds, softmax_scale, qk8)
    out = lse = None
    if poison:
        out = torch.full((B, H, N, v.shape[-1]), float("nan"), dtype=q.dtype, device=dev)
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    o, lse = tara.attn_fwd(qd, kd, vd, seg, tim, pic, mask if use_mask else None, params, out=out, lse=lse)
    torch.cuda.synchronize()
    if poison:
        # rows without any key contribution (none in these workloads) would hold LSE -inf, still not NaN
        bad_o = int(torch.isnan(o).sum())
        bad_l = int(torch.isnan(lse).sum())
        log(f"poisoned outputs after the call: {bad_o} NaN of {o.numel()} O elements, "
            f"{bad_l} NaN of {lse.numel()} LSE elements")
        assert bad_o == 0 and bad_l == 0, "the call left poisoned (unwritten) output elements"
        assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    del qd, kd, vd
    if heads is not None:
        hi = torch.tensor(list(heads), device=dev)
        o, lse = o.index_select(1, hi), lse.index_select(1, hi)
    if rows is not None:
        ri = torch.as_tensor(np.asarray(rows), device=dev)
        o, lse = o.index_select(2, ri), lse.index_select(2, ri)
    return o.float().cpu(), lse.cpu()


def run_oracle(q, k, v, lay: ti.Layout, p: ti.Params, rows=None, heads: Optional[Sequence[int]] = None,
               softmax_scale=None, use_mask=True, key_range=None):
    """fp64 oracle on the same inputs. Returns O [B, Hs, R, D], LSE [B, Hs, R]."""
    B, H, N, D = q.shape
    hs = list(range(H)) if heads is None else list(heads)
    pf = p.f32()
    R = N if rows is None else len(rows)
    o = np.zeros((B, len(hs), R, v.shape[-1]))
    lse = np.zeros((B, len(hs), R))
    mask = lay.mask if use_mask else None
    for b in range(B):
        for i, h in enumerate(hs):
            o[b, i], lse[b, i] = oracle.attention_head(
                q[b, h].float().numpy(), k[b, h].float().numpy(), v[b, h].float().numpy(),
                lay.seg, lay.time, lay.picture, mask, pf, rows=rows, scale=softmax_scale,
                key_range=key_range)
    return o, lse


def run_oracle_all_heads(q, k, v, lay: ti.Layout, p: ti.Params, heads: Optional[Sequence[int]] = None,
                         workers: int = 8, row_block: int = 32768):
    """run_oracle on every row of the given heads (default all) of batch
    element 0, in jobs of one head and up to row_block query rows on `workers`
    threads of this process (NumPy releases the GIL inside its array loops;
    BLAS shares the host's cores, at most 16, among them while they run). No
    child process is started. Returns O [1, Hs, N, D], LSE [1, Hs, N]."""
    import os
    from concurrent.futures import ThreadPoolExecutor, as_completed

    from threadpoolctl import threadpool_limits

    _, H, N, D = q.shape
    hs = list(range(H)) if heads is None else list(heads)
    workers = max(1, workers)
    blas_threads = max(1, min(16, len(os.sched_getaffinity(0))) // workers)
    pf = p.f32()
    o = np.zeros((1, len(hs), N, v.shape[-1]))
    lse = np.zeros((1, len(hs), N))
    host = {}

    def head(h):
        if h not in host:
            host[h] = tuple(x[0, h].float().numpy() for x in (q, k, v))
        return host[h]

    def job(h, r0, r1):
        qh, kh, vh = head(h)
        return h, r0, r1, oracle.attention_head(qh, kh, vh, lay.seg, lay.time, lay.picture, lay.mask, pf,
                                                rows=np.arange(r0, r1))

    for h in hs:   # host copies made once, before the threads start
        head(h)
    with threadpool_limits(limits=blas_threads, user_api="blas"):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            futs = [ex.submit(job, h, r0, min(N, r0 + row_block)) for h in hs for r0 in range(0, N, row_block)]
            for fut in as_completed(futs):
                h, r0, r1, (oh, lh) = fut.result()
                i = hs.index(h)
                o[0, i, r0:r1], lse[0, i, r0:r1] = oh, lh
                log(f"oracle head {h}: rows {r0}..{r1 - 1} done")
    return o, lse


def compare(o_gpu, lse_gpu, o_ref, lse_ref, tol_o=TOL_O, tol_lse=TOL_LSE, tol_rel=TOL_REL_O, what=""):
    """Element-by-element comparison. tol_o is a number or an array of
    per-element bounds broadcastable to O."""
    og = np.asarray(o_gpu, np.float64)
    lg = np.asarray(lse_gpu, np.float64)
    do = np.abs(og - o_ref)
    dl = np.abs(lg - lse_ref)
    rel = float(np.linalg.norm(og - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    res = dict(max_do=float(do.max()), max_dlse=float(dl.max()), rel_o=rel,
               finite=bool(np.isfinite(og).all() and np.isfinite(lg).all()))
    tol = np.broadcast_to(np.asarray(tol_o, np.float64), do.shape)
    res["max_do_over_gate"] = float((do / tol).max())
    log(f"{what}: max|dO|={res['max_do']:.3e} max|dLSE|={res['max_dlse']:.3e} rel={rel:.3e}"
        f" max |dO|/gate={res['max_do_over_gate']:.3f}")
    assert res["finite"], f"{what}: non-finite output"
    assert (do <= tol).all(), f"{what}: |dO| over its gate (worst |dO|/gate {res['max_do_over_gate']:.3f})"
    assert res["max_dlse"] <= tol_lse, f"{what}: max|dLSE| {res['max_dlse']} > {tol_lse}"
    assert rel <= tol_rel, f"{what}: relative |dO| {rel} > {tol_rel}"
    return res


def rounding_gate(q, k, v, lay: ti.Layout, p: ti.Params, o_ref, **oracle_kw):
    """Per-element O gate for peaky softmax, from the arithmetic. The kernel
    rounds each weight p_j to bf16 (unit roundoff u = 2^-8) before the P.V
    product and normalises by the fp32 sum of the unrounded weights, then
    rounds O to bf16. So |dO| <= u * sum_j w_j |v_j| + u |O| with w the exact
    softmax weights; sum_j w_j |v_j| is the oracle's output with |V| for V.
    The gate doubles that and adds 1e-4 for fp32 accumulation and exp2."""
    a, _ = run_oracle(q, k, v.float().abs(), lay, p, **oracle_kw)
    return 2.0 ** -7 * (a + np.abs(o_ref)) + 1e-4


def qkv_random(B, H, N, D, seed, dtype=torch.bfloat16, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    out = []
    for i in range(3):
        x = torch.randn(B, H, N, D, generator=g)
        if i < 2:
            x = x * scale
        out.append(x.to(dtype))
    return tuple(out)


def dequantized(q, k, heads=None, rows=None):
    """fp32 copies of q and k ([B, H, N, D]) with the given heads' K tiles and
    Q rows (all rows when rows is None) replaced by their 8-bit values
    (exact in fp32: E4M3 values times powers of two)."""
    qd, kd = q.float().clone(), k.float().clone()
    hs = range(q.shape[1]) if heads is None else heads
    for b in range(q.shape[0]):
        for h in hs:
            qs = q[b, h].float().numpy() if rows is None else q[b, h, rows].float().numpy()
            a, c = oracle.qk8_dequantize(qs, k[b, h].float().numpy())
            if rows is None:
                qd[b, h] = torch.from_numpy(a).float()
            else:
                qd[b, h, rows] = torch.from_numpy(a).float()
            kd[b, h] = torch.from_numpy(c).float()
    return qd, kd
