"""Calls on several streams and from several host threads at once, through the
C ABI: the library keeps no state between calls beyond the thread-local
error and run info, and its kernels are deterministic (no atomics, a fixed
summation order), so each result must be bit-identical to the same call made
alone on the default stream. One sequential result per case is also checked
against the fp64 oracle.
"""
import threading

import numpy as np
import pytest
import torch

import tara_inputs as ti
import temporally_biased_flashattention_amd as tara
from tara_testlib import compare, device_meta, log, qkv_random, run_oracle, tara_params

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cases():
    out = []
    for i, (n, d, mode) in enumerate([(700, 128, "fused"), (1100, 64, "three-term"), (900, 128, "partitioned"),
                                      (500, 64, "fused")]):
        rng = np.random.default_rng(9700 + i)
        lay = ti.random_layout(rng, n, frames=7, pictures=3, mask=True, shuffle=bool(i % 2))
        p = ti.random_params(rng, 3, binding=True)
        q, k, v = qkv_random(1, 2, n, d, seed=9710 + i)
        out.append((lay, p, mode, q, k, v))
    return out


def _device_inputs(case):
    lay, p, mode, q, k, v = case
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    seg, tim, pic, mask = device_meta(lay)
    params = tara_params(p, mode=mode, partitions=3)
    nbytes = tara.tara_workspace_bytes(tara.TARA_BF16, 1, q.shape[1], q.shape[2], q.shape[3], params)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    return qd, kd, vd, seg, tim, pic, mask, params, ws


def _call(inp):
    qd, kd, vd, seg, tim, pic, mask, params, ws = inp
    return tara.attn_fwd(qd, kd, vd, seg, tim, pic, mask, params, workspace=ws)


def test_streams_and_threads_match_sequential():
    cases = _cases()
    inputs = [_device_inputs(c) for c in cases]
    ref, ref_info = [], []
    for inp in inputs:
        o, l = _call(inp)
        torch.cuda.synchronize()
        ref.append((o.clone(), l.clone()))
        ref_info.append(tara.tara_get_last_run_info())
    assert len({(r["mode"], r["grid"]) for r in ref_info}) == len(ref_info)
    lay, p, mode, q, k, v = cases[0]
    ro, rl = run_oracle(q, k, v, lay, p)
    compare(ref[0][0].float().cpu().numpy(), ref[0][1].cpu().numpy(), ro, rl, what="sequential case 0")

    # all cases enqueued back to back, each on its own stream
    streams = [torch.cuda.Stream() for _ in inputs]
    outs = [None] * len(inputs)
    for i, (inp, s) in enumerate(zip(inputs, streams)):
        with torch.cuda.stream(s):
            outs[i] = _call(inp)
    torch.cuda.synchronize()
    for i, ((o, l), (ro_, rl_)) in enumerate(zip(outs, ref)):
        assert torch.equal(o, ro_) and torch.equal(l, rl_), f"stream case {i} differs from the sequential call"
    log(f"{len(inputs)} cases on {len(streams)} streams: bit-identical")

    # the same from host threads, each with its own stream, three calls each
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    o, l = _call(inputs[i])
                    streams[i].synchronize()
                    if not (torch.equal(o, ref[i][0]) and torch.equal(l, ref[i][1])):
                        errors.append(f"thread {i}: result differs from the sequential call")
                    if tara.tara_get_last_run_info() != ref_info[i]:
                        errors.append(f"thread {i}: run info of another thread's call")
        except Exception as e:  # noqa: BLE001 (reported below)
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(inputs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    log(f"{len(threads)} host threads x 3 calls: bit-identical, run info per thread")
