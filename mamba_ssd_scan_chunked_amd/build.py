"""Build the HIP library libssd_mi355x.so in-tree with hipcc for gfx950.

Usage: python -m mamba_ssd_scan_chunked_amd.build   (or call build()).
Compiles each source to an object in parallel, then links the shared library
next to this file, where the Python binding loads it from.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libssd_mi355x.so")
SOURCES = ["ssd_api.cpp", "ssd_bwd_api.cpp", "ssd_bf16.hip", "ssd_f32.hip"] + [
    "ssd_%s_s%d_e%d_l%d.hip" % (t, sq, eu, lo) for t in ("bf16", "f32") for sq in (0, 1) for eu in (0, 1)
    for lo in (0, 1)] + ["ssd_bwd_bf16.hip", "ssd_bwd_f32.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
            # packed fp32 ops stay off: the kernels use plain fp32 VALU code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-Wall"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + common_flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    msgs = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (src, "\n".join(msgs)))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
