"""Ahead-of-time build of the gfx950 SSD library (libssd.so, in-tree).

    python -m selective_state_space_mamba2_amd.build [--verbose]

Host C++ (metadata builder, validation) is compiled with g++; the HIP sources with hipcc
for gfx950 only.  Packed-fp32 instruction selection is switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libssd.so")

HIP_SOURCES = ["ssd_entry.hip", "ssd_prefill.hip", "ssd_decode.hip", "ssd_diag.hip", "ssd_conv.hip",
               "ssd_debug.hip", "ssd_probe.hip"]
HOST_SOURCES = ["ssd_host.cpp"]
ARCH = "gfx950"
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature name; that warning is expected
    noise = [ln for ln in (res.stderr or "").splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if verbose and noise:
        print("\n".join(noise))


def build(verbose: bool = False) -> str:
    """Compile every source and link libssd.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    jobs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", *inc, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [os.path.join(BUILD, s + ".o") for s in HOST_SOURCES + HIP_SOURCES]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
