"""Seeded synthetic inputs for TARA attention (no attention arithmetic here).

This module is the only code shared by the CPU oracle's tests, the GPU parity
tests and the benchmark. It builds packed token sequences shaped like the
MiniMax H3 sequences the TARA pages describe (target video, the selected
motion-guide video, reference pictures, text), the per-token metadata the
attention rule reads, and seeded Q/K/V. It computes none of the method: no
penalty, no bias, no softmax.

Segment codes follow the C ABI in include/tara.h:
  0 = target (output video), 1 = selected guide video, 2 = reference picture,
  3 = anything else (text, audio, other videos).

Time grid: latent frame f sits at t = f * 4 / 24 seconds on the shared output
clock (24 fps, 4 video frames per latent frame). The TARA pages ask for 24 fps
on both clips and matching frame windows ("Wiring it" section of the TARA
article); the guide uses the same latent frames as the target, with fewer
tokens per frame when the guide is downscaled. Pictures and text carry no
time: their entry is NaN so that any consumer that reads it shows up.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

SEG_TARGET = 0
SEG_GUIDE = 1
SEG_PICTURE = 2
SEG_OTHER = 3

FPS = 24.0
FRAMES_PER_LATENT = 4.0


@dataclasses.dataclass
class Params:
    """TARA controls plus the reference-binding controls (plain numbers)."""
    window: float = 0.20
    falloff: float = 0.25
    strength: float = 2.0
    cap: float = 6.0
    binding: bool = False
    gains: Sequence[float] = ()          # gain per 0-based picture id
    # further bindings applied together with the first (chained binding
    # nodes): one gain tuple per extra binding, same picture ids
    chained: Sequence[Sequence[float]] = ()

    @property
    def num_bindings(self) -> int:
        return 1 + len(self.chained)

    def all_gains(self):
        """Gain tuples of every binding, the first binding first."""
        return (tuple(self.gains),) + tuple(tuple(g) for g in self.chained)

    def f32(self) -> "Params":
        """The same controls rounded to fp32, as a GPU receives them."""
        r = lambda x: float(np.float32(x))
        return Params(r(self.window), r(self.falloff), r(self.strength), r(self.cap),
                      bool(self.binding), tuple(r(g) for g in self.gains),
                      tuple(tuple(r(g) for g in c) for c in self.chained))


@dataclasses.dataclass
class Layout:
    """Per-token metadata of one packed sequence (batch element)."""
    seg: np.ndarray          # uint8 [N]
    time: np.ndarray         # float32 [N], NaN where the token has no time
    picture: np.ndarray      # int16 [N], picture id for pictures, -1 elsewhere
    frame: np.ndarray        # int32 [N], latent frame for video tokens, -1 elsewhere
    # float32 mask weight m of target tokens: [N] for one binding, [J, N] for J
    # chained bindings (one plane per binding); None means m = 1 everywhere
    mask: Optional[np.ndarray] = None

    @property
    def n(self) -> int:
        return int(self.seg.shape[0])

    def permuted(self, perm: np.ndarray) -> "Layout":
        return Layout(self.seg[perm].copy(), self.time[perm].copy(), self.picture[perm].copy(),
                      self.frame[perm].copy(),
                      None if self.mask is None else self.mask[..., perm].copy())


def frame_time(f: np.ndarray) -> np.ndarray:
    """Seconds of latent frame f on the output clock, rounded to fp32."""
    return (np.asarray(f, dtype=np.float64) * FRAMES_PER_LATENT / FPS).astype(np.float32)


def mask_blob(frames: int, rows: int, cols: int, seed: int = 5000, sub: int = 8) -> np.ndarray:
    """Soft mask per latent frame on a rows x cols patch grid, values in (0, 1].

    A smooth Gaussian blob whose centre drifts over the clip, evaluated on
    sub x sub sample points per patch and area-averaged to the patch grid
    (the binding page says soft masks are area-downsampled to the target patch
    resolution). Returns float32 [frames, rows, cols].
    """
    rng = np.random.default_rng(seed)
    phx, phy = rng.uniform(0.0, 2.0 * math.pi, size=2)
    sx, sy = 0.15, 0.20
    off = (np.arange(sub) + 0.5) / sub
    xs = (np.arange(cols)[:, None] + off[None, :]).reshape(-1) / cols   # [cols*sub]
    ys = (np.arange(rows)[:, None] + off[None, :]).reshape(-1) / rows   # [rows*sub]
    out = np.empty((frames, rows, cols), dtype=np.float32)
    for f in range(frames):
        a = 2.0 * math.pi * f / max(frames, 1)
        cx = 0.5 + 0.3 * math.sin(a + phx)
        cy = 0.5 + 0.25 * math.cos(a + phy)
        gx = np.exp(-0.5 * ((xs - cx) / sx) ** 2)
        gy = np.exp(-0.5 * ((ys - cy) / sy) ** 2)
        fine = gy[:, None] * gx[None, :]                                 # [rows*sub, cols*sub]
        out[f] = fine.reshape(rows, sub, cols, sub).mean(axis=(1, 3))
    return out


def shot_length_ok(frames: int) -> bool:
    """True for a prepared shot length of 17n + 5 frames (n >= 0), padding
    included: the only multi-frame mask length the binding page accepts
    ("BFS H3 Reference Attention Binding (Experimental)", "Common issues")."""
    return isinstance(frames, (int, np.integer)) and frames >= 5 and (frames - 5) % 17 == 0


def _area_weights(src: int, dst: int) -> np.ndarray:
    """[dst, src] weights of area resampling: output cell i covers the source
    interval [i*src/dst, (i+1)*src/dst) and averages the source cells it
    overlaps, each weighted by the length of the overlap. Rows sum to 1."""
    e = np.arange(dst + 1, dtype=np.float64) * (src / dst)
    p = np.arange(src, dtype=np.float64)
    ov = np.minimum(e[1:, None], p[None, :] + 1.0) - np.maximum(e[:-1, None], p[None, :])
    return np.clip(ov, 0.0, None) / (src / dst)


def latent_spans(frames: int, latent_frames: int) -> List[tuple]:
    """Pixel frames [lo, hi) averaged into each latent frame: the shot's
    frames split into latent_frames consecutive spans of near-equal length
    (each at least one frame; with one frame, every latent frame takes it)."""
    spans = []
    for j in range(latent_frames):
        lo = j * frames // latent_frames
        hi = max(lo + 1, (j + 1) * frames // latent_frames)
        spans.append((min(lo, frames - 1), min(hi, frames)))
    return spans


def prepare_target_mask(mask, shot_frames: int, latent_frames: int, grid: tuple) -> np.ndarray:
    """Mask weight m of every target token from a soft pixel-space mask.

    mask: [F, height, width] (or [height, width], one static mask) with
    F = 1 or F = shot_frames, the prepared shot length (17n + 5 frames at
    24 fps, padding included); anything else raises ValueError, as a whole-clip
    mask fed to one shot does on the binding page ("BFS H3 Reference Attention
    Binding (Experimental)", "Common issues"). The mask marks output positions.

    Each frame is area-downsampled to the target patch grid (rows, cols), then
    the frames of each latent frame's span (latent_spans) are averaged (the
    same page, "The exact rule": soft masks are area-downsampled to the target
    patch resolution and averaged over the latent temporal spans). Returns
    float32 [latent_frames * rows * cols] in the packed target order
    (frame-major, patches row-major), the per-token mask of the C ABI.
    """
    if not shot_length_ok(shot_frames):
        raise ValueError(f"shot length {shot_frames}: a prepared shot has 17n + 5 frames, padding included")
    m = np.asarray(mask, dtype=np.float64)
    if m.ndim == 2:
        m = m[None]
    if m.ndim != 3 or min(m.shape) < 1:
        raise ValueError("mask must be [frames, height, width] or [height, width]")
    frames = m.shape[0]
    if frames not in (1, shot_frames):
        raise ValueError(f"mask length {frames}: one frame or exactly the shot's {shot_frames} frames")
    if not np.isfinite(m).all():
        raise ValueError("mask values must be finite")
    rows, cols = grid
    if latent_frames < 1 or rows < 1 or cols < 1:
        raise ValueError("latent_frames and the patch grid must be positive")
    ar = _area_weights(m.shape[1], rows)
    ac = _area_weights(m.shape[2], cols)
    small = np.einsum("ip,fpq,jq->fij", ar, m, ac)   # [F, rows, cols]
    out = np.empty((latent_frames, rows, cols), np.float64)
    for j, (lo, hi) in enumerate(latent_spans(frames, latent_frames)):
        out[j] = small[lo:hi].mean(axis=0)
    return out.reshape(-1).astype(np.float32)


def make_layout(frames: int, target_hw: tuple, guide_hw: tuple, pictures: int,
                picture_tokens: int, text: int, mask: bool = False,
                mask_seed: int = 5000, mask_planes: int = 1) -> Layout:
    """Packed sequence [target | guide | pictures by id | text], frame-major.

    target_hw / guide_hw are the (rows, cols) patch grid per latent frame;
    both clips cover the same latent frames. With mask=True every target
    token gets the blob weight of its patch (others get 0); mask_planes > 1
    gives one plane per chained binding, plane j drawn with seed mask_seed + j
    (the mask is then [mask_planes, N]).
    """
    tr, tc = target_hw
    gr, gc = guide_hw
    nt, ng = frames * tr * tc, frames * gr * gc
    npic = pictures * picture_tokens
    n = nt + ng + npic + text
    seg = np.empty(n, np.uint8)
    frame = np.full(n, -1, np.int32)
    pic = np.full(n, -1, np.int16)
    seg[:nt] = SEG_TARGET
    frame[:nt] = np.repeat(np.arange(frames), tr * tc)
    seg[nt:nt + ng] = SEG_GUIDE
    frame[nt:nt + ng] = np.repeat(np.arange(frames), gr * gc)
    seg[nt + ng:nt + ng + npic] = SEG_PICTURE
    pic[nt + ng:nt + ng + npic] = np.repeat(np.arange(pictures), picture_tokens).astype(np.int16)
    seg[nt + ng + npic:] = SEG_OTHER
    time = np.full(n, np.nan, np.float32)
    vid = frame >= 0
    time[vid] = frame_time(frame[vid])
    m = None
    if mask:
        m = np.zeros((mask_planes, n), np.float32)
        for j in range(mask_planes):
            m[j, :nt] = mask_blob(frames, tr, tc, seed=mask_seed + j).reshape(-1)
        if mask_planes == 1:
            m = m[0]
    return Layout(seg, time, pic, frame, m)


def frame_loop_bounds(lay: Layout) -> List[int]:
    """Query-row ranges of a per-frame loop: one range per run of target rows
    of one latent frame, and one per run of the other rows between them.
    Returns the offsets [0, ..., N]."""
    key = np.where(lay.seg == SEG_TARGET, lay.frame.astype(np.int64), -1)
    cuts = np.nonzero(key[1:] != key[:-1])[0] + 1
    return [0] + [int(c) for c in cuts] + [lay.n]


@dataclasses.dataclass
class Config:
    cid: int
    name: str
    heads: int
    head_dim: int
    dtype: str               # "f32" or "bf16"
    layout_args: dict
    params: Params

    def layout(self) -> Layout:
        return make_layout(**self.layout_args)

    @property
    def n(self) -> int:
        a = self.layout_args
        return (a["frames"] * (a["target_hw"][0] * a["target_hw"][1] + a["guide_hw"][0] * a["guide_hw"][1])
                + a["pictures"] * a["picture_tokens"] + a["text"])

    def seed(self, head: int) -> int:
        return 1000 * self.cid + head


def _cfg(cid, name, heads, d, dtype, frames, thw, ghw, pics, ptok, text, params, mask=False, planes=1):
    return Config(cid, name, heads, d, dtype,
                  dict(frames=frames, target_hw=thw, guide_hw=ghw, pictures=pics,
                       picture_tokens=ptok, text=text, mask=mask, mask_planes=planes), params)


# The five workloads: 1 = tiny fp32; 2 = 54,272 tokens x 8 heads; 3 = 107,126 tokens
# x 8 heads (the isolated microbenchmark shape the TARA article reports); 4 = guide
# at scale 0.5 (11,984 guide rows) x 56 heads; 5 = TARA plus reference binding x 56
# heads. 3 with 56 heads is the headline throughput workload (id 6 here).
_CONFIGS = {
    1: _cfg(1, "tiny-fp32-240tok-2h-d64", 2, 64, "f32", 6, (4, 4), (4, 4), 1, 16, 32, Params()),
    2: _cfg(2, "bf16-54272tok-8h-d128", 8, 128, "bf16", 27, (24, 40), (24, 40), 2, 960, 512, Params()),
    3: _cfg(3, "bf16-107126tok-8h-d128", 8, 128, "bf16", 107, (17, 29), (17, 29), 2, 556, 512, Params()),
    4: _cfg(4, "bf16-66359tok-56h-d128-guide0.5", 56, 128, "bf16", 107, (17, 29), (8, 14), 2, 556, 512,
            Params()),
    5: _cfg(5, "bf16-107682tok-56h-d128-binding", 56, 128, "bf16", 107, (17, 29), (17, 29), 3, 556, 512,
            Params(window=0.10, falloff=0.40, strength=3.0, cap=8.0, binding=True,
                   gains=(1.25, 0.75, 0.75)), mask=True),
    6: _cfg(3, "bf16-107126tok-56h-d128", 56, 128, "bf16", 107, (17, 29), (17, 29), 2, 556, 512, Params()),
    # 5's sequence with a second, chained binding (its own mask blob and gains)
    7: _cfg(5, "bf16-107682tok-56h-d128-chained2", 56, 128, "bf16", 107, (17, 29), (17, 29), 3, 556, 512,
            Params(window=0.10, falloff=0.40, strength=3.0, cap=8.0, binding=True,
                   gains=(1.25, 0.75, 0.75), chained=((0.8, 1.4, 1.1),)), mask=True, planes=2),
    # the headline sequence at head dim 64 with twice the heads (the same model
    # width H*D = 7,168 and the same attention FLOP)
    8: _cfg(3, "bf16-107126tok-112h-d64", 112, 64, "bf16", 107, (17, 29), (17, 29), 2, 556, 512, Params()),
}


def config(cid: int) -> Config:
    """Workload by id (1..5; 6 = the 107,126-token layout at 56 heads; 7 = 5
    with a second chained binding; 8 = 6 at head dim 64 with 112 heads)."""
    return _CONFIGS[cid]


def qkv_head(n: int, d: int, seed: int, dtype: str = "bf16"):
    """Q, K, V of one head as CPU torch tensors [n, d] drawn from N(0, 1).

    One torch.Generator seeded with `seed` draws Q, then K, then V in fp32;
    bf16 inputs are the round-to-nearest casts of those draws.
    """
    import torch
    g = torch.Generator().manual_seed(int(seed))
    out = []
    for _ in range(3):
        x = torch.randn(n, d, generator=g, dtype=torch.float32)
        out.append(x.to(torch.bfloat16) if dtype == "bf16" else x)
    return tuple(out)


def qkv(cfg: Config, heads: Optional[Sequence[int]] = None, scale: float = 1.0):
    """Q, K, V for the listed heads of a workload: CPU tensors [1, H, N, D]."""
    import torch
    hs = list(range(cfg.heads)) if heads is None else list(heads)
    n, d = cfg.n, cfg.head_dim
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q = torch.empty(1, len(hs), n, d, dtype=tdt)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    for i, h in enumerate(hs):
        g = torch.Generator().manual_seed(cfg.seed(h))
        for t in (q, k, v):
            x = torch.randn(n, d, generator=g, dtype=torch.float32)
            if scale != 1.0 and t is not v:
                x = x * scale
            t[0, i].copy_(x.to(tdt))
    return q, k, v


def random_params(rng: np.random.Generator, pictures: int, binding: Optional[bool] = None) -> Params:
    """Random but valid controls, for property and brute-force checks."""
    b = bool(rng.integers(0, 2)) if binding is None else binding
    return Params(window=float(rng.uniform(0.0, 0.5)), falloff=float(rng.uniform(0.05, 0.6)),
                  strength=float(rng.uniform(0.0, 4.0)), cap=float(rng.uniform(0.0, 10.0)),
                  binding=b, gains=tuple(float(x) for x in rng.uniform(0.3, 2.5, size=pictures)))


def random_layout(rng: np.random.Generator, n: int, frames: int = 5, pictures: int = 2,
                  mask: bool = True, shuffle: bool = True) -> Layout:
    """A small sequence with all four segment kinds in random proportions/order."""
    cuts = np.sort(rng.integers(0, n + 1, size=3))
    counts = np.diff(np.concatenate([[0], cuts, [n]]))
    seg = np.repeat(np.arange(4, dtype=np.uint8), counts)
    frame = np.full(n, -1, np.int32)
    vid = seg <= SEG_GUIDE
    frame[vid] = rng.integers(0, frames, size=int(vid.sum()))
    pic = np.full(n, -1, np.int16)
    isp = seg == SEG_PICTURE
    pic[isp] = rng.integers(0, max(pictures, 1), size=int(isp.sum())).astype(np.int16)
    time = np.full(n, np.nan, np.float32)
    time[vid] = frame_time(frame[vid])
    m = None
    if mask:
        m = np.zeros(n, np.float32)
        ist = seg == SEG_TARGET
        m[ist] = rng.uniform(0.0, 1.0, size=int(ist.sum())).astype(np.float32)
    lay = Layout(seg, time, pic, frame, m)
    if shuffle:
        lay = lay.permuted(rng.permutation(n))
    return lay


def sample_rows(lay: Layout, n_random: int = 256, per_segment: int = 64, seed: int = 0, tail: int = 64):
    """Stratified query rows: first/last token of each target frame, random
    target rows, random rows from each other segment, and the last rows."""
    rng = np.random.default_rng(seed)
    n = lay.n
    rows = set()
    tgt = np.nonzero(lay.seg == SEG_TARGET)[0]
    if tgt.size:
        fr = lay.frame[tgt]
        for f in np.unique(fr):
            idx = tgt[fr == f]
            rows.add(int(idx[0]))
            rows.add(int(idx[-1]))
        rows.update(int(x) for x in rng.choice(tgt, size=min(n_random, tgt.size), replace=False))
    for s in (SEG_GUIDE, SEG_PICTURE, SEG_OTHER):
        idx = np.nonzero(lay.seg == s)[0]
        if idx.size:
            rows.update(int(x) for x in rng.choice(idx, size=min(per_segment, idx.size), replace=False))
    rows.update(range(max(0, n - tail), n))
    return np.array(sorted(rows), dtype=np.int64)
