"""Builds libserq.so in-tree with hipcc for gfx950.

Usage: ``python -m rank_error_compensated_amd._build`` (or call ``build()``).
The library lands in ``rank_error_compensated_amd/_lib/``; it is what the
Python binding, the tests and the bench load.
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
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libserq.so")
PEAKS_LIB = os.path.join(LIBDIR, "libserq_peaks.so")

SOURCES = ["serq_host.cpp", "serq_kernels.hip"]
PEAKS_SOURCES = ["serq_peaks.hip"]   # the sustained-rate probes the bench reports beside the published peaks

# -ffp-contract=off: every fp32 step that decides a code is one IEEE operation
# (no silent FMA contraction); fp32 division and sqrt stay correctly rounded.
# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 are generated.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-pthread", "-ffp-contract=off", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = ["-x", "hip", "--offload-arch=gfx950", "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the SERQ library needs ROCm's hipcc to build")


def _link(sources, lib: str, verbose: bool) -> str:
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in sources:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc] + (DEVICE if src.endswith(".hip") else []) + ["-c", path, "-o", obj] + COMMON
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = lib + ".tmp"
    cmd = [cc, "-shared", "-o", tmp] + objs + ["--offload-arch=gfx950", "-fPIC", "-pthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile every source and link libserq.so (and the peak probes'
    libserq_peaks.so); returns libserq.so's path."""
    os.makedirs(LIBDIR, exist_ok=True)
    _link(PEAKS_SOURCES, PEAKS_LIB, verbose)
    return _link(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
