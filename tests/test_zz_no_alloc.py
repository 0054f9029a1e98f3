"""cat_forward_1d_noalloc (the 1D forward on the library's fixed device
scratch, for callers that cannot allocate) against cat_forward_1d on the same
inputs, through the C ABI.  The two run the same kernels on the same inputs,
so their outputs must agree bit for bit (stricter than the parity bars); the
smaller case is also checked against the oracle at its storage bar."""
import sys

import numpy as np
import pytest

import oracle
from circulant_softmax_attention_amd import workloads as W
from helpers import assert_parity, ensure_lib, to_dev, to_np

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def cat():
    ensure_lib()
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from circulant_softmax_attention_amd import cat as c
    return c


def _pair(cat, wl):
    import torch
    inp = W.make_inputs(wl)
    plan = cat.cat_plan_create("1d", wl.dtype, wl.B, wl.N, wl.D, wl.H)
    X, WA, WV = (to_dev(a, wl.dtype) for a in (inp.X, inp.W_A, inp.W_V))
    ref = cat.cat_forward_1d(plan, X, WA, WV)
    got = cat.cat_forward_1d_noalloc(plan, X, WA, WV)
    torch.cuda.synchronize()
    return inp, plan, ref, got


def test_noalloc_two_calls_second_smaller(cat):
    """The headline shape (bf16, matrix-core conv), then a smaller fp32
    problem on the vector path at a prime length: each call's output equals
    cat_forward_1d's, and the second call's leftovers from the first (the
    array keeps the last call's contents) change nothing."""
    import torch
    wl1 = W.WORKLOADS["cat1d_gpt2_n1024"]
    say("noalloc", wl1.name)
    _, _, ref1, got1 = _pair(cat, wl1)
    assert torch.equal(ref1, got1)
    wl2 = W.Workload("adhoc", "1d", 2, 197, 96, 3, "f32", 71)
    say("noalloc", wl2)
    inp2, _, ref2, got2 = _pair(cat, wl2)
    assert torch.equal(ref2, got2)
    assert_parity(to_np(got2), oracle.cat_forward_1d(inp2.X, inp2.W_A, inp2.W_V)["O"], "f32", "O")
    # the first call's output is the caller's own buffer and stays intact
    assert torch.equal(ref1, got1)


def test_noalloc_direct_and_long_paths(cat):
    """The direct product (bf16, N <= 256) and the three-pass long path (its
    intermediates also live in the array)."""
    import torch
    for wl in (W.Workload("adhoc", "1d", 4, 200, 128, 2, "bf16", 72),
               W.Workload("adhoc", "1d", 1, 8192, 64, 2, "f32", 73)):
        say("noalloc", wl)
        _, plan, ref, got = _pair(cat, wl)
        assert plan.conv_path() in ("direct", "fft_multipass")
        assert torch.equal(ref, got)


def test_noalloc_rejects_oversize_and_wrong_kind(cat):
    """A problem whose intermediates exceed the fixed array (the CLIP-L layer
    in fp32: 64 MiB of V alone) is refused before any launch, as is a 2D
    plan; an empty batch is a no-op."""
    import torch
    wl = W.WORKLOADS["cat1d_clipL_n256_f32"]
    plan = cat.cat_plan_create("1d", "f32", wl.B, wl.N, wl.D, wl.H)
    x = torch.zeros((wl.B, wl.N, wl.D), device="cuda")
    with pytest.raises(cat.CatError) as e:
        cat.cat_forward_1d_noalloc(plan, x, torch.zeros((wl.D, wl.H), device="cuda"),
                                   torch.zeros((wl.D, wl.D), device="cuda"), O=torch.empty_like(x))
    assert e.value.status == -2
    p2 = cat.cat_plan_create("2d", "f32", 1, 64, 16, 2, Hg=8, Wg=8)
    x2 = torch.zeros((1, 64, 16), device="cuda")
    with pytest.raises(cat.CatError) as e:
        cat.cat_forward_1d_noalloc(p2, x2, torch.zeros((16, 2), device="cuda"), torch.zeros((16, 16), device="cuda"))
    assert e.value.status == -5
    p0 = cat.cat_plan_create("1d", "f32", 0, 16, 16, 2)
    cat.cat_forward_1d_noalloc(p0, torch.zeros((0, 16, 16), device="cuda"), torch.zeros((16, 2), device="cuda"),
                               torch.zeros((16, 16), device="cuda"))
