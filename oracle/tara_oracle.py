"""CPU oracle for TARA temporally-biased attention, in fp64.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, links or runs
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg call it. It is plain, slow and written to be checked against the pages by
eye: the full biased score matrix is built (one block of query rows at a time,
rows being independent), then an ordinary softmax and a matrix product.

What it follows (page titles and sections of the TARA sources):
  * "TARA: Native Temporal Alignment for MiniMax H3 References", section
    "The temporal rule": only edges from output-video (target) queries to the
    selected motion video's (guide) keys change; for them
        dt = |t_output - t_guide|
        penalty(dt) = min(strength * (max(dt - window, 0) / falloff)^2, cap)
        score = dot(Q, K) / sqrt(head_dim) - penalty(dt)
    Defaults window 0.20 s, falloff 0.25 s, strength 2.0, cap 6.0.
  * Same article, first section: text, reference audio, pictures and the
    target's own self-attention keep their normal rule.
  * "BFS H3 Reference Attention Binding (Experimental)", section "The exact
    rule": a target query with mask weight m attending a key of Picture i gets
    m * log(gain_i) added to its logit before the shared softmax over all keys;
    section "Inputs you'll set": no mask means m = 1 on the whole output video;
    section "Common issues": chained binding nodes add their log gains, so J
    bindings give sum_j m_j * log(gain_j,i).
  * LSE is the natural-log log-sum-exp of each query row's final logits, the
    quantity FlashAttention-with-LSE returns and the "Three backends" section
    merges across partitions.

Readings where the pages are silent (each listed in the design notes):
  * one joint, non-causal softmax over every key of the packed sequence;
  * 1/sqrt(head_dim) scales Q.K only, never the penalty or the binding term;
  * log is the natural logarithm; gains must be > 0;
  * a key range restricts the softmax to keys [k0, k1) (one partition).

Segment codes are those of the C ABI: 0 target, 1 guide, 2 picture, 3 other.

What pins it (tests/test_oracle_pins.py, P1-P12): closed forms of the
penalty and of Q = 0 attention, reduction to a library softmax attention
when the bias is off, brute force on tiny inputs, the partition merge and
three-term identities, invariances, monotonicity, chained bindings, and the
8-bit rounding against the format's definition; planted mistakes must fail
them. Every function here has such a pin. The pages print no attention
outputs for a worked example, so absolute O and LSE on random inputs are pinned
through these: the library reduction, brute force and the closed forms.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

TARGET, GUIDE, PICTURE, OTHER = 0, 1, 2, 3


# --------------------------------------------------------------------------- rule
def penalty(dt, window: float, falloff: float, strength: float, cap: float):
    """TARA temporal penalty of a time gap (article, "The temporal rule").

    Zero inside the free window, quadratic in (gap - window) / falloff past it,
    never above cap. Vectorised over dt; fp64.
    """
    dt = np.abs(np.asarray(dt, dtype=np.float64))
    x = np.maximum(dt - window, 0.0) / falloff
    return np.minimum(strength * x * x, cap)


def saturation_gap(window: float, falloff: float, strength: float, cap: float) -> float:
    """Gap past which every guide key gets exactly -cap.

    Solving strength * ((dt - window) / falloff)^2 = cap for dt; with the
    defaults this is 0.2 + 0.25 * sqrt(3) = 0.6330 s, the "about 0.633 s" at
    which the article says the local correction goes to zero.
    """
    if strength <= 0.0:
        return math.inf
    return window + falloff * math.sqrt(cap / strength)


def bias_block(seg_q, time_q, mask_q, seg_k, time_k, pic_k, params) -> np.ndarray:
    """Additive logit bias for a block of query rows against keys, fp64 [R, Nk].

    Target-query x guide-key entries get -penalty(|t_q - t_k|). When binding is
    enabled, target-query x picture-key entries get m_q * ln(gain[picture]),
    m_q = 1 when no mask is given; with chained bindings the terms of every
    binding j are added, sum_j m_j,q * ln(gain_j[picture]) (mask_q is then
    [J, R], one plane per binding). Every other entry is 0.
    """
    seg_q = np.asarray(seg_q)
    seg_k = np.asarray(seg_k)
    bm = np.zeros((seg_q.shape[0], seg_k.shape[0]), dtype=np.float64)
    tq = seg_q == TARGET
    if not tq.any():
        return bm
    rows = np.nonzero(tq)[0]
    gk = np.nonzero(seg_k == GUIDE)[0]
    if gk.size:
        dt = (np.asarray(time_q, np.float64)[rows][:, None]
              - np.asarray(time_k, np.float64)[gk][None, :])
        bm[np.ix_(rows, gk)] = -penalty(dt, params.window, params.falloff, params.strength, params.cap)
    if params.binding:
        pk = np.nonzero(seg_k == PICTURE)[0]
        if pk.size:
            ids = np.asarray(pic_k)[pk].astype(np.int64)
            nb = getattr(params, "num_bindings", 1)
            planes = None if mask_q is None else np.asarray(mask_q, np.float64).reshape(nb, -1)
            gain_sets = params.all_gains() if hasattr(params, "all_gains") else (tuple(params.gains),)
            for j, gains in enumerate(gain_sets):
                gains = np.asarray(gains, dtype=np.float64)
                if np.any(gains <= 0.0):
                    raise ValueError("gains must be > 0 (log of the gain)")
                lg = np.log(gains[ids])
                m = np.ones(rows.size) if planes is None else planes[j][rows]
                bm[np.ix_(rows, pk)] += m[:, None] * lg[None, :]
    return bm


# ---------------------------------------------------------------------- attention
def attention_head(q, k, v, seg, time, picture, mask, params,
                   rows: Optional[Sequence[int]] = None,
                   key_range: Optional[Tuple[int, int]] = None,
                   scale: Optional[float] = None,
                   chunk: int = 128) -> Tuple[np.ndarray, np.ndarray]:
    """Biased softmax attention of one head, fp64.

    q, k, v: [N, D] arrays (any float dtype; upcast exactly to fp64).
    seg/time/picture/mask: per-token metadata of the packed sequence [N]
    (mask may be None). rows: the query rows to compute (default all).
    key_range: (k0, k1) restricts the keys to one partition.
    V may be wider or narrower than Q (probe columns). Returns O [R, Dv] and
    natural-log LSE [R], fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    k0, k1 = (0, n) if key_range is None else key_range
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    seg = np.asarray(seg)
    kk, vk = k[k0:k1], v[k0:k1]
    o = np.zeros((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.full(rows.size, -np.inf, dtype=np.float64)
    if k1 <= k0:
        return o, lse
    for s in range(0, rows.size, chunk):
        r = rows[s:s + chunk]
        z = (q[r] @ kk.T) * sc
        z += bias_block(seg[r], np.asarray(time)[r], None if mask is None else np.asarray(mask)[..., r],
                        seg[k0:k1], np.asarray(time)[k0:k1], np.asarray(picture)[k0:k1], params)
        zmax = z.max(axis=1, keepdims=True)
        l = np.log(np.exp(z - zmax).sum(axis=1)) + zmax[:, 0]
        p = np.exp(z - l[:, None])
        o[s:s + chunk] = p @ vk
        lse[s:s + chunk] = l
    return o, lse


def attention(q, k, v, seg, time, picture, mask, params, rows=None, key_range=None,
              scale=None) -> Tuple[np.ndarray, np.ndarray]:
    """Batched form: q, k, v [B, H, N, D]; metadata [B, N] (mask [B, N], [J, B, N] or None).

    Returns O [B, H, R, D] and LSE [B, H, R] in fp64.
    """
    q = np.asarray(q)
    b, h, n, d = q.shape
    r = n if rows is None else len(rows)
    o = np.zeros((b, h, r, np.asarray(v).shape[-1]))
    lse = np.zeros((b, h, r))
    for bi in range(b):
        for hi in range(h):
            o[bi, hi], lse[bi, hi] = attention_head(
                q[bi, hi], k[bi, hi], v[bi, hi], seg[bi], time[bi], picture[bi],
                None if mask is None else np.asarray(mask)[..., bi, :], params, rows=rows,
                key_range=key_range, scale=scale)
    return o, lse


def merge_partitions(parts) -> Tuple[np.ndarray, np.ndarray]:
    """Exact merge of per-partition results (O_p, LSE_p) over disjoint key sets.

    LSE = ln sum_p exp(LSE_p); O = sum_p exp(LSE_p - LSE) * O_p. Empty
    partitions (LSE_p = -inf) contribute nothing.
    """
    lses = np.stack([p[1] for p in parts])          # [P, R]
    m = lses.max(axis=0)
    lse = m + np.log(np.exp(lses - m).sum(axis=0))
    o = sum(np.exp(l - lse)[:, None] * op for op, l in parts)
    return o, lse


# -------------------------------------------------------- three-term partitions
def three_term_parts(q, k, v, seg, time, picture, mask, params, rows=None, scale=None):
    """The three non-negative contributions of the Flash Partitions backend.

    "TARA: Native Temporal Alignment for MiniMax H3 References", section
    "Three backends": the rule is evaluated by FlashAttention with LSE outputs,
    merging three non-negative contributions instead of building a dense bias
    tensor. Reading (section "The temporal rule": the penalty reaches cap at
    the saturation gap and stays there): with G the guide keys (empty when the
    temporal bias is off, strength or cap 0),
      A: keys outside G, with their normal logits (binding term included);
      B: keys in G, every target row at -cap (other rows unbiased);
      C: keys in G for target rows, weight e^s (e^-penalty - e^-cap) >= 0,
         zero past the saturation gap.
    Returns [(O_A, LSE_A), (O_B, LSE_B), (O_C, LSE_C)] in fp64 (an empty term
    has LSE -inf and O 0); merge_partitions of them is attention_head.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    seg = np.asarray(seg)
    tm = np.asarray(time, np.float64)
    bias_on = params.strength > 0.0 and params.cap > 0.0
    g = (seg == GUIDE) if bias_on else np.zeros(n, bool)
    s = (q[rows] @ k.T) * sc
    full = s + bias_block(seg[rows], tm[rows], None if mask is None else np.asarray(mask)[..., rows],
                          seg, tm, np.asarray(picture), params)
    tgt = seg[rows] == TARGET

    def softmax_part(z):
        # rows with no finite logit give an empty term
        o = np.zeros((rows.size, v.shape[1]))
        lse = np.full(rows.size, -np.inf)
        zmax = z.max(axis=1)
        ok = np.isfinite(zmax)
        if ok.any():
            zz = z[ok] - zmax[ok, None]
            l = np.log(np.exp(zz).sum(axis=1)) + zmax[ok]
            w = np.exp(z[ok] - l[:, None])
            o[ok] = w @ v
            lse[ok] = l
        return o, lse

    za = np.where(g[None, :], -np.inf, full)
    zb = np.where(g[None, :], s - np.where(tgt, params.cap, 0.0)[:, None], -np.inf)
    # term C as a logit: s + ln(e^-p - e^-cap) on (target row, guide key) pairs
    pen = np.zeros_like(s)
    if g.any():
        pen[:, g] = penalty(tm[rows][:, None] - tm[g][None, :], params.window, params.falloff,
                            params.strength, params.cap)
    with np.errstate(divide="ignore"):
        corr = np.log(np.maximum(np.exp(-pen) - math.exp(-params.cap), 0.0))
    zc = np.where(g[None, :] & tgt[:, None], s + corr, -np.inf)
    return [softmax_part(za), softmax_part(zb), softmax_part(zc)]


# ------------------------------------------------------------- 8-bit Q.K (fp8)
# The pages name a dense INT8 one-pass variant of the kernel ("Three
# backends") but give no quantisation scheme; this is the scheme the 8-bit
# Q.K mode uses (a reading, stated in the design notes): OCP FP8 E4M3 values,
# round to nearest even, with a power-of-two scale per query row and per
# 64-key tile of a head, 2^(floor(log2 max|x|) - 7), so the largest magnitude
# lands in [128, 256). Attention then runs on the dequantised Q and K.
E4M3_MAX = 448.0


def fp8_e4m3_round(x):
    """Round to the nearest FP8 E4M3 value (ties to even); |x| <= 448 expected.

    E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; normals from 2^-6,
    subnormals in steps of 2^-9. Rounding is to a multiple of the value's ulp,
    2^(floor(log2|x|) - 3) for normals and 2^-9 below 2^-6.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0.0, a, 1.0)))
    ulp = 2.0 ** (np.maximum(e, -6.0) - 3.0)
    return np.sign(x) * np.round(a / ulp) * ulp          # np.round rounds half to even


def pow2_scale(amax: float) -> float:
    """Power-of-two scale putting amax into [128, 256): 2^(floor(log2 amax) - 7)."""
    if not amax > 0.0:
        return 1.0
    m, e = math.frexp(amax)            # amax = m * 2^e, m in [0.5, 1)
    return math.ldexp(1.0, e - 1 - 7)


def qk8_dequantize(q, k, tile: int = 64):
    """Q and K as the 8-bit Q.K product sees them: each Q row and each tile of
    `tile` consecutive K rows scaled by its power-of-two scale, rounded to
    E4M3 and scaled back. fp64 [N, D] each."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    qd = np.empty_like(q)
    for i in range(q.shape[0]):
        s = pow2_scale(float(np.abs(q[i]).max()))
        qd[i] = fp8_e4m3_round(q[i] / s) * s
    kd = np.empty_like(k)
    for t0 in range(0, k.shape[0], tile):
        blk = k[t0:t0 + tile]
        s = pow2_scale(float(np.abs(blk).max()))
        kd[t0:t0 + tile] = fp8_e4m3_round(blk / s) * s
    return qd, kd


# -------------------------------------------------------------------- brute force
def attention_bruteforce(q, k, v, seg, time, picture, mask, params, scale=None):
    """Pure-Python loops with exactly rounded sums, for tiny inputs (N <= ~32).

    Same definition as attention_head, written element by element: logit,
    bias, exp, fsum, weighted sum.
    """
    n = len(q)
    d = len(q[0])
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out_o, out_l = [], []
    for i in range(n):
        zs = []
        for j in range(n):
            z = math.fsum(float(q[i][c]) * float(k[j][c]) for c in range(d)) * sc
            if int(seg[i]) == TARGET and int(seg[j]) == GUIDE:
                dt = abs(float(time[i]) - float(time[j]))
                x = max(dt - params.window, 0.0) / params.falloff
                z -= min(params.strength * x * x, params.cap)
            if params.binding and int(seg[i]) == TARGET and int(seg[j]) == PICTURE:
                gain_sets = params.all_gains() if hasattr(params, "all_gains") else (tuple(params.gains),)
                for b, gains in enumerate(gain_sets):
                    if mask is None:
                        m = 1.0
                    else:
                        mk = np.asarray(mask)
                        m = float(mk[i]) if mk.ndim == 1 else float(mk[b][i])
                    z += m * math.log(gains[int(picture[j])])
            zs.append(z)
        zm = max(zs)
        lse = zm + math.log(math.fsum(math.exp(z - zm) for z in zs))
        w = [math.exp(z - lse) for z in zs]
        out_o.append([math.fsum(w[j] * float(v[j][c]) for j in range(n)) for c in range(d)])
        out_l.append(lse)
    return np.array(out_o), np.array(out_l)
