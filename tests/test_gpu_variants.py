"""GPU parity of the averaged-key and causal variants of CAT, called through
the C ABI, against the fp64 CPU oracle on the same seeded inputs.

Bars: fp32 storage -> relative L2 <= 1e-5 and max-abs <= 1e-4; bf16
storage -> relative L2 <= 2e-2.  The averaged-key logits are computed in
fp32 from the stored inputs, so they meet the fp32 bar in both dtypes.
"""
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


def avgkey_inputs(seed, B, N, D, H, dtype):
    wl = W.Workload("adhoc", "1d", B, N, D, H, dtype, seed)
    inp = W.make_inputs(wl)
    WQ, WK = W.extra_square_weights(wl, 2)
    return inp, WQ, WK


# ------------------------------------------------------------------ averaged-key
@pytest.mark.parametrize("B,N,D,H,dtype", [(1, 64, 64, 4, "f32"), (2, 37, 48, 3, "f32"), (3, 100, 64, 4, "bf16"),
                                           (1, 1, 32, 2, "f32"), (2, 197, 384, 6, "f32"), (1, 1024, 768, 12, "bf16"),
                                           (2, 130, 136, 17, "bf16"), (1, 300, 2048, 32, "f32"),
                                           (2, 65, 3072, 24, "bf16")])
def test_avgkey_logits(cat, B, N, D, H, dtype):
    """The logits alone, every token, against the oracle's definition
    (Q and K formed, token-mean key, / sqrt(d)).  Ragged token blocks,
    H not a multiple of 4, D across several 1024-slices and the largest D."""
    say("avgkey_logits", B, N, D, H, dtype)
    import torch
    inp, WQ, WK = avgkey_inputs(41, B, N, D, H, dtype)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    z = cat.cat_step_avgkey_logits(plan, to_dev(inp.X, dtype), to_dev(WQ, dtype), to_dev(WK, dtype))
    torch.cuda.synchronize()
    ref = oracle.avgkey_scores_1d(inp.X, WQ, WK, H)
    # scale-aware: the logits' size shrinks like N^-1/2 for random inputs, so
    # the fp32 bar is applied relative to their largest entry (never looser
    # than the stated 1e-4)
    sc = float(np.max(np.abs(ref)))
    assert_parity(to_np(z) / max(sc, 1.0), ref / max(sc, 1.0), "f32", "z")


@pytest.mark.parametrize("B,N,D,H,dtype,path", [
    (2, 64, 64, 4, "f32", "fft_valu"), (1, 1024, 128, 2, "bf16", "fft_matrix"), (2, 200, 128, 2, "bf16", "direct"),
    (3, 197, 96, 3, "f32", "fft_valu"), (1, 1, 32, 2, "f32", "fft_valu"), (1, 2048, 64, 2, "bf16", "fft_valu")])
def test_forward_avgkey_1d(cat, B, N, D, H, dtype, path):
    """The whole averaged-key forward on every single-workgroup mixing path."""
    say("forward_avgkey_1d", B, N, D, H, dtype, path)
    import torch
    inp, WQ, WK = avgkey_inputs(43, B, N, D, H, dtype)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    assert plan.conv_path() == path
    O = cat.cat_forward_avgkey_1d(plan, to_dev(inp.X, dtype), to_dev(WQ, dtype), to_dev(WK, dtype),
                                  to_dev(inp.W_V, dtype))
    torch.cuda.synchronize()
    assert_parity(to_np(O), oracle.cat_avgkey_forward_1d(inp.X, WQ, WK, inp.W_V, H)["O"], dtype, "O")


@pytest.mark.parametrize("N,dtype", [(8192, "f32"), (6000, "bf16")])
def test_forward_avgkey_1d_long(cat, N, dtype):
    """The averaged-key forward on the three-pass mixing, 512 sampled rows."""
    B, D, H = 1, 64, 2
    say("forward_avgkey_1d_long", B, N, D, H, dtype)
    import torch
    inp, WQ, WK = avgkey_inputs(47, B, N, D, H, dtype)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    assert plan.conv_path() == "fft_multipass"
    O = cat.cat_forward_avgkey_1d(plan, to_dev(inp.X, dtype), to_dev(WQ, dtype), to_dev(WK, dtype),
                                  to_dev(inp.W_V, dtype))
    torch.cuda.synchronize()
    rows = np.unique(np.random.default_rng(5).integers(0, B * N, 512))
    ref = oracle.cat_avgkey_forward_1d(inp.X, WQ, WK, inp.W_V, H, rows=rows)["O"]
    assert_parity(to_np(O).reshape(B * N, D)[rows], ref, dtype, "O rows")


def test_forward_avgkey_1d_workload_full_size(cat):
    """The averaged-key forward at the GPT-2-small layer shape (B = 16,
    N = 1024, D = 768, H = 12, bf16; the workload's X and W_V, W_Q and W_K
    drawn by the same recipe), on the launch configuration of the headline;
    the oracle checks three whole sequences."""
    import torch
    wl = W.WORKLOADS["cat1d_gpt2_n1024"]
    say("forward_avgkey_full", wl.name)
    inp = W.make_inputs(wl)
    WQ, WK = W.extra_square_weights(wl, 2)
    plan = cat.cat_plan_create("1d", wl.dtype, wl.B, wl.N, wl.D, wl.H)
    O = to_np(cat.cat_forward_avgkey_1d(plan, to_dev(inp.X, wl.dtype), to_dev(WQ, wl.dtype), to_dev(WK, wl.dtype),
                                        to_dev(inp.W_V, wl.dtype)))
    torch.cuda.synchronize()
    for b in (0, 7, wl.B - 1):
        ref = oracle.cat_avgkey_forward_1d(inp.X[b:b + 1], WQ, WK, inp.W_V, wl.H)["O"]
        assert_parity(O[b:b + 1], ref, wl.dtype, f"b={b}")


def test_avgkey_rejections(cat):
    import torch
    p2 = cat.cat_plan_create("2d", "f32", 1, 64, 16, 2, Hg=8, Wg=8)
    x = torch.zeros((1, 64, 16), device="cuda")
    w = torch.zeros((16, 16), device="cuda")
    with pytest.raises(cat.CatError) as e:
        cat.cat_forward_avgkey_1d(p2, x, w, w, w)
    assert e.value.status == -5
    big = cat.cat_plan_create("1d", "bf16", 1, 8, 4096, 32)
    xb = torch.zeros((1, 8, 4096), device="cuda", dtype=torch.bfloat16)
    wb = torch.zeros((4096, 4096), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(cat.CatError) as e:
        cat.cat_forward_avgkey_1d(big, xb, wb, wb, wb)
    assert e.value.status == -2


# ------------------------------------------------------------------ causal
@pytest.mark.parametrize("B,N,D,H", [(1, 1, 32, 1), (2, 2, 64, 2), (1, 17, 64, 2), (2, 31, 64, 1), (1, 32, 128, 4),
                                     (2, 33, 64, 2), (1, 100, 96, 3), (2, 197, 64, 2), (1, 255, 64, 1),
                                     (3, 256, 128, 2)])
@pytest.mark.parametrize("scale", [2.0, 1e-3, 12.0])
def test_mix_causal_1d(cat, B, N, D, H, scale):
    """The causal mixing alone from logits: N = 1, 2, primes, the ends of the
    32-token steps and the longest line; near-uniform (scale 1e-3), ordinary
    and peaked (scale 12) logits."""
    say("mix_causal_1d", B, N, D, H, scale)
    import torch
    rng = np.random.default_rng(N * 5 + D)
    logits = (rng.standard_normal((B, H, N)) * scale).astype(np.float32)
    V = rng.standard_normal((B, N, D)).astype(np.float32)
    V = W.bf16_bits_to_f32(W.round_bf16_bits(V)).reshape(V.shape)
    plan = cat.cat_plan_create("1d", "bf16", B, N, D, H)
    O = cat.cat_step_mix_causal_1d(plan, torch.from_numpy(logits).cuda(), to_dev(V, "bf16"))
    torch.cuda.synchronize()
    ref = oracle.causal_1d(logits, V)
    got = to_np(O)
    assert_parity(got, ref, "bf16", "O")
    # row 0 of every head is V[0]: its one weight is divided by itself (the
    # normalisers sum the bf16-rounded weights the products use), so only the
    # fp32 reciprocal's rounding is left, below the output's bf16 rounding
    assert np.allclose(got[:, 0], V[:, 0], rtol=2 ** -8, atol=0)


@pytest.mark.parametrize("B,N,D,H", [(2, 64, 64, 2), (3, 100, 64, 2), (1, 197, 384, 6), (2, 256, 128, 4)])
def test_forward_causal_1d(cat, B, N, D, H):
    say("forward_causal_1d", B, N, D, H)
    import torch
    wl = W.Workload("adhoc", "1d", B, N, D, H, "bf16", 53)
    inp = W.make_inputs(wl)
    plan = cat.cat_plan_create("1d", "bf16", B, N, D, H)
    O = cat.cat_forward_causal_1d(plan, to_dev(inp.X, "bf16"), to_dev(inp.W_A, "bf16"), to_dev(inp.W_V, "bf16"))
    torch.cuda.synchronize()
    assert_parity(to_np(O), oracle.cat_causal_forward_1d(inp.X, inp.W_A, inp.W_V)["O"], "bf16", "O")


def test_forward_causal_1d_workload_full_size(cat):
    """Causal CAT at the CLIP-L layer shape (B = 64, N = 256, D = 1024,
    H = 16, bf16 storage, the workload's inputs); the oracle checks the first
    and the last image in full."""
    import torch
    wl = W.WORKLOADS["cat1d_clipL_n256_bf16"]
    say("forward_causal_full", wl.name)
    inp = W.make_inputs(wl)
    plan = cat.cat_plan_create("1d", wl.dtype, wl.B, wl.N, wl.D, wl.H)
    O = to_np(cat.cat_forward_causal_1d(plan, to_dev(inp.X, wl.dtype), to_dev(inp.W_A, wl.dtype),
                                        to_dev(inp.W_V, wl.dtype)))
    torch.cuda.synchronize()
    for b in (0, wl.B - 1):
        ref = oracle.cat_causal_forward_1d(inp.X[b:b + 1], inp.W_A, inp.W_V)["O"]
        assert_parity(O[b:b + 1], ref, wl.dtype, f"b={b}")


def test_causal_rejections(cat):
    """Outside the direct product's range the call is refused before any
    launch."""
    import torch
    for (dtype, N, D, H) in [("f32", 64, 64, 2), ("bf16", 257, 64, 2), ("bf16", 64, 48, 3)]:
        dt = torch.float32 if dtype == "f32" else torch.bfloat16
        plan = cat.cat_plan_create("1d", dtype, 1, N, D, H)
        x = torch.zeros((1, N, D), device="cuda", dtype=dt)
        with pytest.raises(cat.CatError) as e:
            cat.cat_forward_causal_1d(plan, x, torch.zeros((D, H), device="cuda", dtype=dt),
                                      torch.zeros((D, D), device="cuda", dtype=dt))
        assert e.value.status == -2
