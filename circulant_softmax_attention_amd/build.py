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
# The matrix-core conv reads every MFMA result with vector ALU instructions;
# asking the backend for MFMAs that write VGPRs directly saves a copy of each
# result out of the accumulation registers.
FILE_FLAGS = {"cat_mconv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
SOURCES = ["cat_inst_2d_96.hip", "cat_inst_2d_vit.hip", "cat_inst_1d_large.hip", "cat_inst_1d_mid.hip", "cat_inst_2d_small.hip",
           "cat_inst_1d_small.hip", "cat_gemm.hip", "cat_mconv.hip", "cat_dconv.hip", "cat_longconv.hip", "cat_fftconv.hip", "cat_backward.hip", "cat_variants.hip", "cat_noalloc.hip", "cat_bconv.hip", "cat_score96.hip",
           "cat_api.cpp"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE_FLAGS
    cmd += FILE_FLAGS.get(src, [])
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


def _stale(src: str) -> bool:
    """True when the object of `src` is missing or older than the source or
    any header it may include (every header of csrc/ and include/)."""
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)]
    for d, ext in ((CSRC, ".hpp"), (os.path.join(ROOT, "include"), ".h")):
        deps += [os.path.join(d, f) for f in os.listdir(d) if f.endswith(ext)]
    return os.path.getmtime(obj) < max(os.path.getmtime(f) for f in deps)


def build(verbose: bool = True, only=None) -> str:
    """Compile every source (or the sources named in `only` plus every source
    whose object is out of date, reusing the other objects) and link
    libcat.so."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    todo = SOURCES if not only else [s for s in SOURCES if s in only or _stale(s)]
    if verbose:
        print(f"building {LIB} for {ARCH} ({len(todo)} of {len(SOURCES)} sources)", flush=True)
    with cf.ThreadPoolExecutor(max_workers=len(todo)) as ex:
        list(ex.map(lambda s: _compile(s, verbose), todo))
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"objects missing (run a full build): {missing}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, only=sys.argv[1:] or None)
    sys.exit(0)
