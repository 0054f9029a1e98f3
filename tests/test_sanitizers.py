"""Host sanitizer builds (AddressSanitizer and UndefinedBehaviorSanitizer)
of the fp64 oracle and of the C ABI's host code, run on the CPU.

The oracle is compiled with gcc and driven through every function on small
ragged inputs (tests/sanitize/oracle_driver.c).  The ABI's host file
(cat_api.cpp: problem validation, geometry, workspace layout, host tables,
error paths) is compiled with the sanitizers on its host side only (each
-fsanitize= right after -Xarch_host; device code is not instrumented),
linked with the library's other objects and driven through every
validation path (tests/sanitize/abi_driver.cpp).  Without a GPU, plan
creation stops at its first device call; with one, the plans are built and
destroyed.  Any sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
SAN_FLAGS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def _clean(out):
    return "AddressSanitizer" not in out and "runtime error" not in out and "LeakSanitizer" not in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-std=c11", *SAN_FLAGS,
                    os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "cat_oracle.c"), "-lm",
                    "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=dict(ENV, OMP_NUM_THREADS="2"), timeout=300)
    assert rc == 0 and _clean(out), out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_host_code_under_sanitizers(tmp_path):
    from circulant_softmax_attention_amd import build as B
    # the library's other objects (compiled only where missing or stale)
    B.build(verbose=False, only=["cat_api.cpp"])
    objs = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "cat_api.cpp"]
    host_san = [f for flag in SAN_FLAGS for f in ("-Xarch_host", flag)]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", B.CSRC]
    api_o, drv_o, exe = str(tmp_path / "cat_api_san.o"), str(tmp_path / "abi_driver.o"), str(tmp_path / "abi_driver")
    common = [HIPCC, "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", f"--offload-arch={B.ARCH}", *inc]
    rc, out = _run(common + host_san + ["-c", os.path.join(B.CSRC, "cat_api.cpp"), "-o", api_o])
    assert rc == 0, out
    rc, out = _run(common + host_san + ["-c", os.path.join(SAN, "abi_driver.cpp"), "-o", drv_o])
    assert rc == 0, out
    rc, out = _run([HIPCC, f"--offload-arch={B.ARCH}", *host_san, drv_o, api_o, *objs, "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=300)
    assert rc == 0 and _clean(out), out
    assert "all expectations held" in out
