"""Builds libssm.so (the gfx950 HIP kernels and the C-ABI host layer) in-tree.

    python -m selective_state_space_68_amd.build_lib

Each translation unit is compiled with hipcc for gfx950 only, then linked into
selective_state_space_68_amd/libssm.so.  Packed-fp32 instruction selection is
disabled for device code (-packed-fp32-ops); the host pass warns that it does
not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libssm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
DEVICE_SOURCES = ["scan_sequential.hip", "scan_chunked.hip", "state_update.hip", "conv1d.hip", "scan_bwd.hip", "ssd.hip", "scan_tokseq.hip", "calib.hip", "ssd_noalloc.hip"]
HOST_SOURCES = ["ssm_api.cpp"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n  " + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, f"--offload-arch={ARCH}", *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
