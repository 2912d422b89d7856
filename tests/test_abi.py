"""C-ABI checks that need no GPU: the library loads, exports what include/tara.h
declares, sizes workspaces, and rejects bad arguments on the host (argument
errors are detected before any device work, so these calls never reach HIP)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import temporally_biased_flashattention_amd as tara

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tara.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tara_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return tara.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), f"{n} declared in tara.h but not exported"
    assert sorted(tara.EXPORTED_SYMBOLS) == names


def test_missing_library_fails_loudly(tmp_path):
    """Without the built library every entry point raises; there is no fallback."""
    import sys
    code = ("import temporally_biased_flashattention_amd as t\n"
            "for f in (t.load_library, t.tara_params_default):\n"
            "    try:\n"
            "        f()\n"
            "    except t.TaraLibraryMissing as e:\n"
            "        print('missing:', f.__name__)\n"
            "    else:\n"
            "        raise SystemExit(f.__name__ + ' did not raise')\n")
    env = dict(os.environ, TARA_LIBRARY=str(tmp_path / "absent.so"), PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("missing:") == 2


def test_params_struct_matches_header_defaults():
    p = tara.tara_params_default()
    assert (p.window, p.falloff, p.strength, p.cap) == pytest.approx((0.20, 0.25, 2.0, 6.0))
    assert p.binding_enabled == 0 and p.mode == tara.TARA_MODE_FUSED and p.num_partitions == 1
    assert p.num_bindings == 1
    assert all(p.picture_gain[j][i] == 1.0 for j in range(4) for i in range(16))
    assert p.softmax_scale == 0.0
    assert p.qk8 == 0
    # ctypes layout: 4 floats, 3 ints, 4x16 floats, float, 2 ints, pointer, int (+4 padding)
    assert ctypes.sizeof(tara.TaraParams) == 4 * 4 + 3 * 4 + 64 * 4 + 4 + 2 * 4 + 8 + 8


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_run_info_layout_matches_c(tmp_path):
    """The ctypes mirror of tara_run_info_t has the C compiler's size and offsets."""
    fields = [n for n, _ in tara.TaraRunInfo._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"tara.h\"\nint main(void) {\n"
                   + "".join(f'  printf("%zu\\n", offsetof(tara_run_info_t, {n}));\n' for n in fields)
                   + '  printf("%zu\\n", sizeof(tara_run_info_t));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = [getattr(tara.TaraRunInfo, n).offset for n in fields] + [ctypes.sizeof(tara.TaraRunInfo)]
    assert got == want


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_params_layout_matches_c(tmp_path):
    """The ctypes mirror of tara_params_t has the C compiler's size and offsets."""
    fields = [n for n, _ in tara.TaraParams._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"tara.h\"\nint main(void) {\n"
                   + "".join(f'  printf("%zu\\n", offsetof(tara_params_t, {n}));\n' for n in fields)
                   + '  printf("%zu\\n", sizeof(tara_params_t));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = [getattr(tara.TaraParams, n).offset for n in fields] + [ctypes.sizeof(tara.TaraParams)]
    assert got == want


def _al(x):
    return (x + 255) // 256 * 256


def test_workspace_bytes():
    p = tara.tara_params_default()
    B, H, N, D = 1, 2, 1000, 128
    npad = 1024
    nkt = npad // 64
    ngroups = (N + 31) // 32     # tile-class counts: 5 per group of 32 query rows
    meta = _al(B * N * 4) + 2 * _al(B * npad * 4) + _al(0) + _al(B * nkt * 16) + _al(B * ngroups * 5 * 4)
    bf16_extra = _al(B * H * D * npad * 2) + _al(B * H * nkt * 4)     # V^T, per-tile max |k|
    assert tara.tara_workspace_bytes(tara.TARA_BF16, B, H, N, D, p) == meta + bf16_extra
    assert tara.tara_workspace_bytes(tara.TARA_FP32, B, H, N, D, p) == meta
    pp = tara.make_params(mode="partitioned", partitions=3)
    assert tara.tara_workspace_bytes(tara.TARA_BF16, B, H, N, D, pp) == (
        meta + bf16_extra + _al(3 * B * H * N * D * 4) + _al(3 * B * H * N * 4))
    p3 = tara.make_params(mode="three-term")
    assert tara.tara_workspace_bytes(tara.TARA_BF16, B, H, N, D, p3) == (
        meta + bf16_extra + _al(3 * B * H * N * D * 4) + _al(3 * B * H * N * 4))
    pb = tara.make_params(binding=True, gains=(1.25, 0.75, 0.75), chained=((0.9, 1.1, 1.0),))
    assert tara.tara_workspace_bytes(tara.TARA_FP32, B, H, N, D, pb) == meta + _al(B * N * 3 * 4)   # gain table
    assert tara.tara_workspace_bytes(tara.TARA_BF16, 0, H, N, D, p) == 0
    p8 = tara.make_params(qk8=True)   # FP8 keys [B*H][npad][D] and one scale per key tile
    assert tara.tara_workspace_bytes(tara.TARA_BF16, B, H, N, D, p8) == (
        meta + bf16_extra + _al(B * H * npad * D) + _al(B * H * nkt * 4))
    with pytest.raises(tara.TaraError):
        tara.tara_workspace_bytes(tara.TARA_FP32, B, H, N, D, p8)
    with pytest.raises(tara.TaraError):
        tara.tara_workspace_bytes(tara.TARA_BF16, B, H, N, D, tara.make_params(qk8=True, mode="three-term"))
    # baselines: a dense fp32 bias [B][N][npad]; the frame loop needs nothing extra
    pdb = tara.make_params(mode="dense-bias")
    assert tara.tara_workspace_bytes(tara.TARA_BF16, B, H, N, D, pdb) == meta + bf16_extra + _al(B * N * npad * 4)
    with pytest.raises(tara.TaraError):
        tara.tara_workspace_bytes(tara.TARA_FP32, B, H, N, D, pdb)
    pfl = tara.make_params(mode="frame-loop", partitions=7)
    assert tara.tara_workspace_bytes(tara.TARA_BF16, B, H, N, D, pfl) == meta + bf16_extra
    assert tara.tara_workspace_bytes(tara.TARA_FP32, B, H, N, D, pfl) == meta
    with pytest.raises(tara.TaraError):
        tara.tara_workspace_bytes(tara.TARA_BF16, 1, 1, 10, 96, p)
    with pytest.raises(tara.TaraError):
        tara.tara_workspace_bytes(7, 1, 1, 10, 64, p)


# --------------------------------------------------------------- rejections
FAKE = 0x10000          # never dereferenced: every call below fails host checks first


def call(lib, params, dtype=tara.TARA_BF16, B=1, H=2, N=100, D=128, q=FAKE, k=FAKE, v=FAKE, o=FAKE,
         lse=FAKE, strides=None, seg=FAKE, time=FAKE, pic=FAKE, mask=0, ws=FAKE, ws_bytes=1 << 40):
    if strides is None:
        strides = (H * N * D, N * D, D)
    s = [(ctypes.c_int64 * 3)(*strides) for _ in range(4)]
    return lib.tara_attn_fwd(q, k, v, o, lse, dtype, B, H, N, D, s[0], s[1], s[2], s[3],
                             seg, time, pic, mask or None, ctypes.byref(params) if params is not None else None,
                             ws, ws_bytes, None)


def test_rejections(lib):
    P = tara.tara_params_default
    assert call(lib, None) == -1
    assert call(lib, P(), dtype=5) == -3
    assert call(lib, P(), D=96) == -4
    assert call(lib, P(), N=-1) == -2
    assert call(lib, P(), B=300, H=300) == -2
    assert call(lib, P(), q=0) == -1
    assert call(lib, P(), seg=0) == -1
    assert call(lib, P(), q=FAKE + 8) == -5                      # base not 16-byte aligned
    assert call(lib, P(), strides=(1000 * 128, 100 * 128, 130)) == -5   # row stride not x8
    assert call(lib, P(), dtype=tara.TARA_FP32, strides=(800, 400, 6)) == -5
    # bf16: one head's key rows are addressed with 32-bit byte offsets
    # (row stride x N padded to 64, and D x N padded, below 2^31 bytes)
    # (ws_bytes=10: a call that passes these checks stops at the workspace check)
    n = 1 << 20
    assert call(lib, P(), H=8, N=n, strides=(n * 8 * 128, 128, 8 * 128), ws_bytes=10) == -5   # BNHD, 8 heads: 2^31
    assert call(lib, P(), H=7, N=n, strides=(n * 7 * 128, 128, 7 * 128), ws_bytes=10) == -7   # 7 heads: below
    assert call(lib, P(), N=(1 << 23) - 10, H=1, ws_bytes=10) == -5                          # D x Npad x 2 = 2^31
    assert call(lib, P(), N=(1 << 23) - 64, H=1, ws_bytes=10) == -7                          # one tile less
    assert call(lib, P(), ws_bytes=10) == -7
    assert call(lib, P(), ws=0) == -7
    assert call(lib, P(), ws=FAKE + 64) == -7                    # not 256-byte aligned
    assert call(lib, tara.make_params(falloff=0.0)) == -6
    assert call(lib, tara.make_params(falloff=-1.0)) == -6
    assert call(lib, tara.make_params(window=-0.1)) == -6
    assert call(lib, tara.make_params(strength=-1.0)) == -6
    assert call(lib, tara.make_params(cap=-1.0)) == -6
    assert call(lib, tara.make_params(cap=float("inf"))) == -6
    assert call(lib, tara.make_params(window=float("nan"))) == -6
    assert call(lib, tara.make_params(binding=True, gains=(1.25, 0.0))) == -6
    assert call(lib, tara.make_params(binding=True, gains=(1.25, -2.0))) == -6
    assert call(lib, tara.make_params(softmax_scale=-1.0)) == -6
    assert call(lib, tara.make_params(binding=True, gains=(1.25, 0.5), chained=((1.0, 0.0),))) == -6
    assert call(lib, tara.make_params(binding=True, gains=(1.25, 0.5), chained=((1.0, float("nan")),))) == -6
    pb = tara.make_params(binding=True, gains=(1.25,))
    pb.num_bindings = 5
    assert call(lib, pb) == -6
    pb.num_bindings = -1
    assert call(lib, pb) == -6
    assert call(lib, tara.make_params(binding=True, gains=(1.25,)), pic=0) == -1   # ids needed
    assert call(lib, tara.make_params(mode="partitioned", partitions=0)) == -6
    assert call(lib, tara.make_params(mode="partitioned", partitions=65)) == -6
    assert call(lib, tara.make_params(mode="partitioned", partitions=2, bounds=(0, 50, 99))) == -6
    assert call(lib, tara.make_params(mode="partitioned", partitions=2, bounds=(0, 60, 50))) == -6
    assert call(lib, tara.make_params(mode="partitioned", partitions=2, bounds=(1, 50, 100))) == -6
    p = P()
    p.mode = 7
    assert call(lib, p) == -6
    # 8-bit Q.K: bf16 and fused mode only
    assert call(lib, tara.make_params(qk8=True), dtype=tara.TARA_FP32, strides=(2 * 100 * 128, 100 * 128, 128)) == -6
    assert call(lib, tara.make_params(qk8=True, mode="partitioned", partitions=2)) == -6
    assert call(lib, tara.make_params(qk8=True, mode="three-term")) == -6
    # baselines
    assert call(lib, tara.make_params(mode="dense-bias"), dtype=tara.TARA_FP32,
                strides=(2 * 100 * 128, 100 * 128, 128)) == -6
    assert call(lib, tara.make_params(mode="frame-loop", partitions=0)) == -6
    assert call(lib, tara.make_params(mode="frame-loop", partitions=101)) == -6          # > N
    assert call(lib, tara.make_params(mode="frame-loop", partitions=2, bounds=(0, 60, 99))) == -6
    assert call(lib, tara.make_params(mode="frame-loop", partitions=2, bounds=(0, 60, 40))) == -6
    assert call(lib, tara.make_params(qk8=True, mode="frame-loop", partitions=2)) == -6
    # three-term passes keep their key-tile lists in LDS: N <= 2^20
    assert call(lib, tara.make_params(mode="three-term"), N=(1 << 20) + 64, H=1) == -2


def test_probe_rejections(lib):
    out = ctypes.c_float(0.0)
    assert lib.tara_probe_mfma_bf16(100, 1, None, None) == -1
    assert lib.tara_probe_mfma_bf16(0, 1, ctypes.byref(out), None) == -6
    assert lib.tara_probe_mfma_bf16((1 << 24) + 1, 0, ctypes.byref(out), None) == -6
    assert lib.tara_probe_mfma_bf16(100, 2, ctypes.byref(out), None) == -6
    assert lib.tara_probe_mfma_bf16(100, -1, ctypes.byref(out), None) == -6


def test_messages(lib):
    call(lib, tara.make_params(falloff=0.0))
    assert "falloff" in tara.tara_last_error()
    for st in range(0, -10, -1):
        assert tara.tara_status_string(st) and tara.tara_status_string(st) != "unknown status"
    assert tara.tara_status_string(-99) == "unknown status"


def test_empty_calls_are_ok_without_device_work(lib):
    # B, H or N == 0: valid, nothing enqueued (no HIP call is made)
    assert call(lib, tara.tara_params_default(), N=0, q=0, k=0, v=0, o=0, lse=0, ws=0) == 0
    assert call(lib, tara.tara_params_default(), B=0, q=0, k=0, v=0, o=0, lse=0, ws=0) == 0
    info = tara.tara_get_last_run_info()
    assert info["launches"] == 0 and info["block_k"] == 64


def test_timing_read_empty(lib):
    tara.tara_timing_enable(False)
    assert tara.tara_timing_read() == []


def test_workspace_bytes_tail_split():
    """A fused bf16 call of 20,020 tokens x 8 heads (79 query blocks of 256
    rows per head: 632 workgroups, 2.5 rounds of 256 compute units) hands rows
    16,384.. to the range pass over two key ranges (with 8-bit Q.K too): the
    workspace holds their partial O and LSE. Other modes, fp32 and calls
    within one round do not."""
    p = tara.tara_params_default()
    B, H, N, D = 1, 8, 20020, 128
    npad = (N + 63) // 64 * 64
    nkt = npad // 64
    ngroups = (N + 31) // 32
    meta = _al(B * N * 4) + 2 * _al(B * npad * 4) + _al(0) + _al(B * nkt * 16) + _al(B * ngroups * 5 * 4)
    base = meta + _al(B * H * D * npad * 2) + _al(B * H * nkt * 4)
    rows = N - 64 * 256
    tail = _al(2 * B * H * rows * D * 4) + _al(2 * B * H * rows * 4)
    assert tara.tara_workspace_bytes(tara.TARA_BF16, B, H, N, D, p) == base + tail
    assert tara.tara_workspace_bytes(tara.TARA_BF16, B, H, N, D, tara.make_params(qk8=True)) == (
        base + _al(B * H * npad * D) + _al(B * H * nkt * 4) + tail)
    assert tara.tara_workspace_bytes(tara.TARA_BF16, B, 1, 2000, D, p) == tara.tara_workspace_bytes(
        tara.TARA_BF16, B, 1, 2000, D, tara.make_params(mode="frame-loop", partitions=1))


def test_tail_split_plan_at_the_benchmark_shapes():
    """The planned tail splits of the benchmark shapes, read off the workspace
    (the partial O and LSE of the split-off rows): at 107,126 tokens x 56
    heads, 3 of 419 query blocks per head (630 rows) in 3 key ranges; at 8
    heads the same rows in 10 key ranges; at 112 heads x d64, 3 key ranges;
    at 9 heads (1,467 blocks left over, more than two rounds) none."""
    p = tara.tara_params_default()
    N = 107126

    def ws(H, D, params=p):
        return tara.tara_workspace_bytes(tara.TARA_BF16, 1, H, N, D, params)

    def partials(H, D, parts, rows=630):
        return _al(parts * H * rows * D * 4) + _al(parts * H * rows * 4)

    unsplit = tara.make_params(mode="frame-loop", partitions=1)   # same regions, never split
    assert ws(56, 128) == ws(56, 128, unsplit) + partials(56, 128, 3)
    assert ws(8, 128) == ws(8, 128, unsplit) + partials(8, 128, 10)
    assert ws(112, 64) == ws(112, 64, unsplit) + partials(112, 64, 3)
    assert ws(9, 128) == ws(9, 128, unsplit)
