"""Build libcat.so (gfx950) in-tree with hipcc.

    python -m circulant_softmax_attention_amd.build      # or build() from Python

Each translation unit is compiled in parallel, then linked into
circulant_softmax_attention_amd/libcat.so.  Device code is built for gfx950
only, with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcat.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-I", CSRC, "-Wall", "-Wno-unused-function"]
SOURCES = ["cat_inst_2d_96.hip", "cat_inst_1d_large.hip", "cat_inst_1d_mid.hip", "cat_inst_2d_small.hip",
           "cat_inst_1d_small.hip", "cat_gemm.hip", "cat_fftconv.hip", "cat_api.cpp"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE_FLAGS
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if verbose:
        print(f"  {src}: {time.time() - t0:.1f}s", flush=True)
        for ln in msgs:
            print("   ", ln)
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link libcat.so; always rebuilds."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    if verbose:
        print(f"building {LIB} for {ARCH}", flush=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
