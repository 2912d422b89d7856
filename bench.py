"""Throughput of TARA attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline|2|3|4|5|7|8]
                    [--mode fused|partitioned|three-term|dense-bias|frame-loop] [--qk8]
                    [--no-tile-skip]

A step is one tara_attn_fwd call (metadata encoding, V layout pass, the fused
attention kernel; in partitioned mode the range passes plus the merge; in
three-term mode the three Flash Partitions passes plus the merge; the
dense-bias baseline writes the whole bias tensor and then reads it; the
frame-loop baseline launches the fused pass once per target latent frame and
once for the other rows) over the whole workload, inputs already resident in HBM. The default workload is the 107,126-token
packed sequence (52,751 target + 52,751 guide + 2 x 556 picture + 512 text
tokens, 107 latent frames) at 56 heads of dim 128 in bf16 with the default
TARA controls. Prints one JSON line. --qk8 takes Q.K in FP8 E4M3 (per-row
and per-key-tile power-of-two scales; P.V stays bf16); its roofline peak is
that of the FLOP mix, half at the FP8 MFMA peak and half at the bf16 one.
--no-tile-skip sends every key tile through the per-element bias (the
library's TARA_DISABLE_TILE_SKIP switch), to measure what the tile classes
buy; the results are the same up to rounding.

Effective work per step is 4 * B * H * N^2 * D FLOP (both products over every
query/key pair; bias skipping removes no contraction work).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk/CU)
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS
# Q.K at the FP8 rate and P.V at the bf16 rate, equal FLOP each
PEAK_QK8_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (256 CU x 2.4 GHz x 256 FLOP/clk/CU), the fp32 path's bound
METRIC = "TARA attention TFLOP/s and % of bf16 MFMA peak at 107,126 tok × 56 heads"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_headline_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "temporally_biased_flashattention_amd", "csrc", "tara_kernels.hip")


def attention_flop(b: int, h: int, rows: int, n: int, d: int) -> float:
    """Effective work of the dense path: both products over every (query row,
    key) pair, 2 FLOP per multiply-add, Q.K^T and P.V each rows * n * d
    multiply-adds per head; bias skipping removes no contraction work."""
    return 4.0 * b * h * rows * n * d


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def workload(name):
    import tara_inputs as ti
    cid = 6 if name == "headline" else int(name)
    return ti.config(cid)


def measured_traffic(workload_name):
    """HBM bytes per attention launch from the committed counter summary, if
    it was taken on the current kernel source and this workload and mode
    (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha() or t.get("workload") != workload_name:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, q, k, v, lay, seconds: float):
    """The fp64 oracle (as it stands) on a bounded, stratified sample of query
    rows of head 0, timed on the host cores; scaled to effective TFLOP/s."""
    import numpy as np

    import oracle
    from tara_inputs import sample_rows
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 0)) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    rows = sample_rows(lay, n_random=30000, per_segment=512, seed=1)
    rng = np.random.default_rng(2)
    rows = rng.permutation(rows)
    qh, kh, vh = (x[0, 0].float().numpy() for x in (q, k, v))
    p = cfg.params.f32()
    done = 0
    t0 = time.perf_counter()
    while done < len(rows) and time.perf_counter() - t0 < seconds:
        r = np.sort(rows[done:done + 128])
        oracle.attention_head(qh, kh, vh, lay.seg, lay.time, lay.picture, lay.mask, p, rows=r)
        done += len(r)
    dt = time.perf_counter() - t0
    flop = attention_flop(1, 1, done, lay.n, cfg.head_dim)
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} stratified query rows of head 0 of {cfg.name} against all {lay.n} keys, "
                      f"fp64 NumPy oracle, {dt:.1f} s",
            "cpu": cpu_model(), "host_cpus": os.cpu_count()}


def cpu_model() -> str:
    """The host CPU's model name (Linux), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class ClockSampler:
    """Samples the GPU's current shader (GFX) clock through amdsmi every
    `period` seconds in a background thread while the timed steps run; the
    clock the chip settles at under the load (it is power-limited) sets how
    much of the nominal peak the kernel can reach. Reports nothing if amdsmi
    is unavailable."""

    def __init__(self, period: float = 0.02):
        self.period = period
        self.samples = []
        self.error = None
        self._stop = None
        self._thread = None
        self._handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self._amdsmi = amdsmi
            self._handle = handles[0] if handles else None
            if self._handle is None:
                self.error = "no GPU handle"
        except Exception as e:  # noqa: BLE001
            self.error = f"amdsmi unavailable: {e}"

    def _read(self):
        info = self._amdsmi.amdsmi_get_clock_info(self._handle, self._amdsmi.AmdSmiClkType.GFX)
        return float(info.get("clk", info.get("cur_clk")))

    def _loop(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception as e:  # noqa: BLE001
                self.error = f"clock read failed: {e}"
                return
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        if self._handle is not None:
            self._stop = threading.Event()
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        if not self.samples:
            return {"median": None, "samples": 0, "source": "amdsmi GFX clock", "error": self.error}
        xs = sorted(self.samples)
        return {"median": xs[len(xs) // 2], "min": xs[0], "max": xs[-1], "samples": len(xs),
                "source": "amdsmi GFX clock, sampled during the timed steps"}


def oracle_configs(seconds: float):
    """Times the fp64 oracle (as it stands) on every workload, on this host's
    cores: workloads 1 and 2 on all rows and heads, the larger ones on a
    bounded stratified row sample of head 0, extrapolated linearly to all
    rows and heads. One JSON line per workload."""
    import numpy as np

    import oracle
    import tara_inputs as ti
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 0)) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    for cid in (1, 2, 3, 4, 5, 6, 7, 8):
        cfg = ti.config(cid)
        lay = cfg.layout()
        n, h, d = lay.n, cfg.heads, cfg.head_dim
        p = cfg.params.f32()
        full = cid in (1, 2)
        t0 = time.perf_counter()
        if full:
            q, k, v = ti.qkv(cfg)
            for hh in range(h):
                oracle.attention_head(q[0, hh].float().numpy(), k[0, hh].float().numpy(), v[0, hh].float().numpy(),
                                      lay.seg, lay.time, lay.picture, lay.mask, p)
            rows, heads = n, h
        else:
            q, k, v = ti.qkv(cfg, heads=[0])
            rs = np.random.default_rng(3).permutation(ti.sample_rows(lay, n_random=30000, per_segment=512, seed=3))
            qh, kh, vh = (x[0, 0].float().numpy() for x in (q, k, v))
            done = 0
            while done < len(rs) and time.perf_counter() - t0 < seconds:
                r = np.sort(rs[done:done + 256])
                oracle.attention_head(qh, kh, vh, lay.seg, lay.time, lay.picture, lay.mask, p, rows=r)
                done += len(r)
            rows, heads = done, 1
        dt = time.perf_counter() - t0
        total = dt * (n / rows) * (h / heads)
        print(json.dumps({"workload": cfg.name, "tokens": n, "heads": h, "head_dim": d,
                          "oracle_s_per_call": round(total, 1), "timed_s": round(dt, 1),
                          "timed": "all rows and heads" if full else f"{rows} stratified rows of head 0, "
                                                                    "extrapolated to all rows and heads",
                          "tflops": round(attention_flop(1, heads, rows, n, d) / dt / 1e12, 4),
                          "cores": cores, "cpu": cpu_model(), "host_cpus": os.cpu_count()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--mode", default="fused",
                    choices=["fused", "partitioned", "three-term", "dense-bias", "frame-loop"])
    ap.add_argument("--partitions", type=int, default=3)
    ap.add_argument("--qk8", action="store_true", help="8-bit Q.K (bf16 workloads, fused mode)")
    ap.add_argument("--no-tile-skip", action="store_true",
                    help="every key tile takes the per-element bias (sets TARA_DISABLE_TILE_SKIP=1)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib-gib", type=float, default=0.0,
                    help="also run a plain device copy of this many GiB (counter calibration)")
    ap.add_argument("--oracle-configs", action="store_true",
                    help="time the fp64 oracle on every workload on this host's cores (no GPU used) and exit")
    args = ap.parse_args()
    if args.oracle_configs:
        oracle_configs(args.cpu_seconds)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus} GPUs, WORLD_SIZE={world}); "
              "TARA attention here is a single-GPU kernel and no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)

    if args.no_tile_skip:
        os.environ["TARA_DISABLE_TILE_SKIP"] = "1"   # read by the library at every call
    import torch

    import tara_inputs as ti
    import temporally_biased_flashattention_amd as tara

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    tara.load_library()
    cfg = workload(args.workload)
    lay = cfg.layout()
    B, H, N, D = 1, cfg.heads, lay.n, cfg.head_dim
    log(f"workload {cfg.name}: N={N} H={H} D={D} dtype={cfg.dtype}; generating inputs")
    t0 = time.perf_counter()
    q, k, v = ti.qkv(cfg)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda", 0)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    seg = torch.from_numpy(lay.seg)[None].to(dev)
    tim = torch.from_numpy(lay.time)[None].to(dev)
    pic = torch.from_numpy(lay.picture)[None].to(dev)
    # mask: [1, N], or [J, 1, N] with one plane per chained binding
    mask = None if lay.mask is None else torch.from_numpy(lay.mask)[..., None, :].contiguous().to(dev)
    cp = cfg.params
    bounds = ti.frame_loop_bounds(lay) if args.mode == "frame-loop" else None
    nparts = len(bounds) - 1 if bounds else args.partitions if args.mode == "partitioned" else 1
    params = tara.make_params(window=cp.window, falloff=cp.falloff, strength=cp.strength, cap=cp.cap,
                              binding=cp.binding, gains=tuple(cp.gains), mode=args.mode,
                              partitions=nparts, bounds=bounds,
                              chained=tuple(tuple(c) for c in cp.chained), qk8=args.qk8)
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(tara.tara_workspace_bytes(tara.TARA_BF16 if cfg.dtype == "bf16" else tara.TARA_FP32,
                                                   B, H, N, D, params), 1), dtype=torch.uint8, device=dev)

    def step():
        tara.tara_attn_fwd(qd, kd, vd, o, lse, seg, tim, pic, mask, params, ws)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")
    tara.tara_timing_read()
    tara.tara_timing_enable(True)
    # per-step HIP events on the stream the library launches on (torch's current one)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        evs[0].record()
        for i in range(args.steps):
            step()
            evs[i + 1].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    tara.tara_timing_enable(False)
    kms = tara.tara_timing_read()
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    log(f"{args.steps} timed steps in {elapsed:.3f} s; step median {step_ms[len(step_ms) // 2]:.3f} ms, "
        f"min {step_ms[0]:.3f} ms; GFX clock {clock.summary()}")
    info = tara.tara_get_last_run_info()
    # the bf16 MFMA rates this box sustains with nothing else to do, right after the timed
    # steps: on varied operands (power-limited, the practical ceiling on real data) and on
    # constant operands (the top clock)
    probe = tara.tara_probe_mfma_bf16(1000000, tara.TARA_PROBE_RANDOM)
    probe_const = tara.tara_probe_mfma_bf16(400000, tara.TARA_PROBE_CONSTANT)
    log(f"MFMA-only probes: {probe:.1f} TFLOP/s on varied operands, {probe_const:.1f} on constant operands")

    if args.copy_calib_gib > 0:
        nb = int(args.copy_calib_gib * (1 << 30))
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {nb} bytes")
        del src, dst

    flop = attention_flop(B, H, N, N, D)
    ms_step = elapsed / args.steps * 1e3
    value = flop / (ms_step / 1e3) / 1e12
    k_avg = sum(kms) / len(kms) if kms else float("nan")
    achieved = flop / (k_avg / 1e3) / 1e12
    traffic = None if args.qk8 or args.no_tile_skip else measured_traffic(f"{cfg.name} {args.mode}")
    # fp32 inputs run the FMA path: bound by the fp32 vector ALUs, not the MFMA units
    fp32_path = cfg.dtype != "bf16"
    peak = PEAK_FP32_VALU_TFLOPS if fp32_path else PEAK_QK8_TFLOPS if args.qk8 else PEAK_BF16_TFLOPS
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (Q.K) + bf16 (P.V)" if args.qk8 else cfg.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, packed H3-shaped metadata)",
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        # each timed step from HIP events around it on the stream (the whole call)
        "step_ms": {"mean": round(ms_step, 3), "median": round(step_ms[len(step_ms) // 2], 3),
                    "min": round(step_ms[0], 3), "max": round(step_ms[-1], 3)},
        "gfx_clock_mhz": clock.summary(),
        "config": {"workload": f"{cfg.name} ({args.mode}{', 8-bit Q.K' if args.qk8 else ''}"
                               f"{', per-element bias on every tile' if args.no_tile_skip else ''})", "tokens": N, "heads": H, "head_dim": D, "batch": B,
                   "target_tokens": int((lay.seg == 0).sum()), "guide_tokens": int((lay.seg == 1).sum()),
                   "mode": args.mode, "partitions": info.get("num_partitions"), "qk8": args.qk8,
                   # false: every key tile took the per-element bias (--no-tile-skip)
                   "tile_skip": not info.get("elem_all"),
                   "controls": {"window": cfg.params.window, "falloff": cfg.params.falloff,
                                "strength": cfg.params.strength, "cap": cfg.params.cap,
                                "binding": cfg.params.binding, "gains": list(cfg.params.gains),
                                "chained_gains": [list(c) for c in cfg.params.chained]},
                   "block_q": info.get("block_q"), "block_k": info.get("block_k"), "grid": info.get("grid"),
                   # fused bf16: the last query blocks of every head run as a range pass over this many
                   # key ranges plus a merge (0: none); the timed attention work includes both
                   "tail_parts": info.get("tail_parts")},
        "roofline": {"bound": "alu" if fp32_path else "mfma", "achieved": round(achieved, 3), "peak": round(peak, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": ("attn_bf16_kernel" + (" (fused pass + tail range pass + merge)" if info.get("tail_parts") else ""))
                               if cfg.dtype == "bf16" else "attn_f32_kernel",
                     "kernel_ms_avg": round(k_avg, 4), "launches_timed": len(kms),
                     "kernel_ms_median": round(sorted(kms)[len(kms) // 2], 4) if kms else None,
                     "kernel_ms_min": round(min(kms), 4) if kms else None,
                     "flop_per_launch": flop,
                     # back-to-back bf16 MFMAs on register operands, same box: varied operands
                     # (power-limited like the kernel's own products) and constant ones
                     "mfma_probe_tflops": round(probe, 1), "frac_of_mfma_probe": round(achieved / probe, 4),
                     "mfma_probe_constant_tflops": round(probe_const, 1)},
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle for about {args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(cfg, q, k, v, lay, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
