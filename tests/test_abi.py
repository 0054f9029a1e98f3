"""The C ABI on the CPU: the library loads, exports what include/cat.h
declares, and rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

from helpers import ROOT, ensure_lib

ensure_lib()
from circulant_softmax_attention_amd import cat  # noqa: E402

HEADER = os.path.join(ROOT, "include", "cat.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cat_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["cat_plan_create", "cat_plan_destroy", "cat_plan_workspace_size",
                     "cat_forward_1d", "cat_forward_bccb_2d", "cat_status_string"]:
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(cat.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(cat.EXPORTS) == declared_functions()


def test_status_strings():
    lib = cat.lib()
    for code, name in cat.STATUS_NAMES.items():
        assert lib.cat_status_string(code).decode() == name


def _create(**kw):
    p = dict(kind=cat.CAT_1D, dtype=cat.CAT_F32, B=2, N=64, D=64, H=4, Hg=0, Wg=0)
    p.update(kw)
    prob = cat._Problem(p["kind"], p["dtype"], p["B"], p["N"], p["D"], p["H"], p["Hg"], p["Wg"])
    h = ctypes.c_void_p(12345)
    st = cat.lib().cat_plan_create(ctypes.byref(h), ctypes.byref(prob))
    return st, h.value


@pytest.mark.parametrize("kw,status", [
    (dict(kind=7), -1),
    (dict(dtype=5), -1),
    (dict(B=-1), -1),
    (dict(N=0), -1),
    (dict(H=0), -1),
    (dict(D=60, H=8), -1),        # D % H != 0
    (dict(D=24, H=8), -1),        # d = 3 is odd
    (dict(D=36, H=2), -1),        # D % 8 != 0
    (dict(kind=cat.CAT_BCCB_2D, N=64, Hg=8, Wg=7), -1),  # Hg*Wg != N
    (dict(kind=cat.CAT_BCCB_2D, N=35, Hg=5, Wg=7), -2),  # grid not instantiated
    (dict(N=32769), -2),          # non-power-of-two beyond 32768
    (dict(N=131072), -2),         # power of two beyond 65536
    (dict(N=40000), -2),          # non-power-of-two beyond 32768
    (dict(D=1024, H=64), -2),     # 1D with more than 32 heads
    (dict(B=1 << 20, N=4096, D=1024), -2),  # B*N*D >= 2^31
])
def test_plan_create_rejects_before_any_hip_call(kw, status):
    st, h = _create(**kw)
    assert st == status
    assert h is None  # *out is cleared
    assert cat.lib().cat_last_error().decode() != ""


def test_null_arguments():
    lib = cat.lib()
    prob = cat._Problem(0, 0, 1, 64, 64, 4, 0, 0)
    assert lib.cat_plan_create(None, ctypes.byref(prob)) == -1
    h = ctypes.c_void_p()
    assert lib.cat_plan_create(ctypes.byref(h), None) == -1
    assert lib.cat_plan_destroy(None) == 0
    n = ctypes.c_size_t()
    assert lib.cat_plan_workspace_size(None, ctypes.byref(n)) == -1
    assert lib.cat_forward_1d(None, None, None, None, None, None, None) == -1
    assert lib.cat_forward_bccb_2d(None, None, None, None, None, None, None, None) == -1
    assert lib.cat_step_mix(None, None, None, None, None, None) == -1


def test_binding_raises_cat_error():
    with pytest.raises(cat.CatError) as e:
        cat.cat_plan_create("1d", "f32", B=1, N=64, D=60, H=8)
    assert e.value.status == -1
