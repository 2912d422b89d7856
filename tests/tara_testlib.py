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
            softmax_scale=0.0, layout="bhnd", use_mask=True, heads=None, rows=None, qk8=False):
    """q, k, v: CPU tensors [B, H, N, D]. Returns (O fp32 CPU, LSE fp32 CPU),
    restricted to the given heads and query rows when those are given."""
    dev = "cuda"
    B = q.shape[0]
    if layout == "bhnd":
        qd, kd, vd = (x.to(dev).contiguous() for x in (q, k, v))
    else:   # stored [B, N, H, D], passed as a [B, H, N, D] view
        qd, kd, vd = (x.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3) for x in (q, k, v))
    seg, tim, pic, mask = device_meta(lay, dev, B)
    params = tara_params(p, mode, partitions, bounds, softmax_scale, qk8)
    o, lse = tara.attn_fwd(qd, kd, vd, seg, tim, pic, mask if use_mask else None, params)
    torch.cuda.synchronize()
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


def compare(o_gpu, lse_gpu, o_ref, lse_ref, tol_o=TOL_O, tol_lse=TOL_LSE, tol_rel=TOL_REL_O, what=""):
    og = np.asarray(o_gpu, np.float64)
    lg = np.asarray(lse_gpu, np.float64)
    do = np.abs(og - o_ref)
    dl = np.abs(lg - lse_ref)
    rel = float(np.linalg.norm(og - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    res = dict(max_do=float(do.max()), max_dlse=float(dl.max()), rel_o=rel,
               finite=bool(np.isfinite(og).all() and np.isfinite(lg).all()))
    log(f"{what}: max|dO|={res['max_do']:.3e} max|dLSE|={res['max_dlse']:.3e} rel={rel:.3e}")
    assert res["finite"], f"{what}: non-finite output"
    assert res["max_do"] <= tol_o, f"{what}: max|dO| {res['max_do']} > {tol_o}"
    assert res["max_dlse"] <= tol_lse, f"{what}: max|dLSE| {res['max_dlse']} > {tol_lse}"
    assert rel <= tol_rel, f"{what}: relative |dO| {rel} > {tol_rel}"
    return res


def qkv_random(B, H, N, D, seed, dtype=torch.bfloat16, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    out = []
    for i in range(3):
        x = torch.randn(B, H, N, D, generator=g)
        if i < 2:
            x = x * scale
        out.append(x.to(dtype))
    return tuple(out)


def sample_rows(lay: ti.Layout, n_random: int = 256, per_segment: int = 64, seed: int = 0, tail: int = 64):
    """Stratified query rows: first/last token of each target frame, random
    target rows, random rows from each other segment, and the last rows."""
    rng = np.random.default_rng(seed)
    n = lay.n
    rows = set()
    tgt = np.nonzero(lay.seg == ti.SEG_TARGET)[0]
    if tgt.size:
        fr = lay.frame[tgt]
        for f in np.unique(fr):
            idx = tgt[fr == f]
            rows.add(int(idx[0]))
            rows.add(int(idx[-1]))
        rows.update(int(x) for x in rng.choice(tgt, size=min(n_random, tgt.size), replace=False))
    for s in (ti.SEG_GUIDE, ti.SEG_PICTURE, ti.SEG_OTHER):
        idx = np.nonzero(lay.seg == s)[0]
        if idx.size:
            rows.update(int(x) for x in rng.choice(idx, size=min(per_segment, idx.size), replace=False))
    rows.update(range(max(0, n - tail), n))
    return np.array(sorted(rows), dtype=np.int64)


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
