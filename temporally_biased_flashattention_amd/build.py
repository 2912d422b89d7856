"""Builds libtara.so (the C-ABI library with the gfx950 kernels) in-tree.

    python -m temporally_biased_flashattention_amd.build

Every source is compiled by hipcc for gfx950 only. Packed-fp32 instruction
selection is turned off for device code (-packed-fp32-ops); hipcc's host pass
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtara.so")
SOURCES = ["tara_kernels.hip", "tara_host.cpp", "tara_probe.hip", "tara_noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libtara.so)")


def common_flags():
    return ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False, jobs: int = 2) -> str:
    """Compiles every source and links libtara.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    for p in procs:
        _wait(p, verbose)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    return LIB


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    noise = "is not a recognized feature for this target"
    text = "\n".join(l for l in out.splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{text}")
    if verbose and text.strip():
        print(text)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
