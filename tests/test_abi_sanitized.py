"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds tests/abi_sanitizer_driver.c with the library sources, host code
instrumented (-Xarch_host before each sanitizer flag: device code is built
as usual and never runs here), and runs it on the CPU: every call in the
driver fails its host checks or is an empty call, so no device work happens.
The run must print ALL OK with no sanitizer report. Leak checking is off:
the HIP runtime keeps allocations until exit that are not this library's.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "temporally_biased_flashattention_amd", "csrc")
SOURCES = ["tara_kernels.hip", "tara_host.cpp", "tara_probe.hip", "tara_noalloc.hip"]
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs ROCm's hipcc and clang")
def test_abi_rejections_under_asan_and_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs, objs = [], []
    for src in SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = ([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + HOST_SAN + inc
               + ["-c", os.path.join(CSRC, src), "-o", obj])
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for pr in procs:
        out, _ = pr.communicate(timeout=600)
        assert pr.returncode == 0, out
    drv = str(tmp_path / "driver.o")
    subprocess.run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(ROOT, "tests", "abi_sanitizer_driver.c"), "-o", drv], check=True, timeout=300)
    exe = str(tmp_path / "driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950"] + HOST_SAN + [drv] + objs + ["-o", exe, "-lm"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=99",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    report = run.stdout + run.stderr
    print(report[-3000:])
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-3000:]
    assert run.returncode == 0 and "ALL OK" in run.stdout, report[-3000:]
    assert "WRONG" not in run.stdout
