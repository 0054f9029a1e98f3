"""GPU parity: every step and the whole forward path, called through the C
ABI, against the fp64 CPU oracle on the same seeded inputs.

Bars (written here, from the workload specification): fp32 storage ->
relative L2 <= 1e-5 and max-abs <= 1e-4; bf16 storage with fp32 compute ->
relative L2 <= 2e-2.  Spectra (an internal quantity with no oracle function)
are checked against numpy's FFT of the oracle's softmax, at the fp32 bar.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from circulant_softmax_attention_amd import workloads as W
from helpers import (as_real_pairs, assert_parity, assert_spectrum_parity, ensure_lib, rel_l2, sum_bar, to_dev,
                     to_np)

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


def rng_inputs(seed, B, N, D, H, dtype, kind="1d", score_scale=1.0):
    wl = W.Workload("adhoc", kind, B, N, D, H, dtype, seed)
    if kind == "2d":
        raise ValueError
    return W.make_inputs(wl, score_scale=score_scale)


def rng_inputs_2d(seed, B, Hg, Wg, D, H, dtype, score_scale=1.0):
    wl = W.Workload("adhoc2d", "2d", B, Hg * Wg, D, H, dtype, seed, Hg=Hg, Wg=Wg)
    return W.make_inputs(wl, score_scale=score_scale)


def tdtype(dtype):
    import torch
    return torch.float32 if dtype == "f32" else torch.bfloat16


# ------------------------------------------------------------------ 1D steps
@pytest.mark.parametrize("B,N,D,H,dtype", [(1, 64, 64, 4, "f32"), (3, 37, 48, 3, "f32"), (2, 200, 136, 17, "bf16"),
                                           (2, 256, 256, 4, "bf16"), (1, 130, 200, 25, "bf16"),
                                           (2, 96, 320, 32, "f32")])
def test_project_1d(cat, B, N, D, H, dtype):
    say("project_1d", B, N, D, H, dtype)
    inp = rng_inputs(11, B, N, D, H, dtype)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    V, z = cat.cat_step_project(plan, to_dev(inp.X, dtype), to_dev(inp.W_A, dtype), to_dev(inp.W_V, dtype))
    import torch
    torch.cuda.synchronize()
    assert_parity(to_np(V), oracle.matmul(inp.X, inp.W_V), dtype, "V")
    assert_parity(to_np(z), oracle.scores_1d(inp.X, inp.W_A), "f32", "z")


@pytest.mark.parametrize("tile_m", [128, 256])
@pytest.mark.parametrize("tile_n", [96, 128, 192])
@pytest.mark.parametrize("B,N,D,H,dtype", [(2, 300, 264, 12, "bf16"), (1, 200, 200, 25, "bf16"),
                                           (2, 300, 264, 6, "bf16"), (1, 520, 256, 16, "bf16"),
                                           (3, 130, 136, 17, "f32")])
def test_project_tile_widths(cat, monkeypatch, tile_m, tile_n, B, N, D, H, dtype):
    """Every output tile shape of the projection GEMM (forced through the
    tuning variables), with ragged rows, a K tail, several column tiles and
    one or two 16-head blocks of the score projection, whose W_A rows are
    read transposed (heads a multiple of 4) or one value at a time.  Shapes a
    case does not allow (192 columns or 256 rows with fp32 operands, 96
    columns with 256 rows, 128 x 192 with the score projection) fall back to
    an allowed one."""
    say("project_tile", tile_m, tile_n, B, N, D, H, dtype)
    monkeypatch.setenv("CAT_GEMM_TILE_N", str(tile_n))
    monkeypatch.setenv("CAT_GEMM_TILE_M", str(tile_m))
    inp = rng_inputs(17, B, N, D, H, dtype)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    V, z = cat.cat_step_project(plan, to_dev(inp.X, dtype), to_dev(inp.W_A, dtype), to_dev(inp.W_V, dtype))
    import torch
    torch.cuda.synchronize()
    assert_parity(to_np(V), oracle.matmul(inp.X, inp.W_V), dtype, "V")
    assert_parity(to_np(z), oracle.scores_1d(inp.X, inp.W_A), "f32", "z")


@pytest.mark.parametrize("tile_m", [128, 256])
@pytest.mark.parametrize("tile_n", [96, 128, 192])
def test_forward_1d_tile_widths(cat, monkeypatch, tile_m, tile_n):
    """The whole 1D path (blocked value layout) at every GEMM tile shape."""
    B, N, D, H, dtype = 2, 160, 384, 6, "bf16"
    say("forward_tile", tile_m, tile_n, B, N, D, H, dtype)
    monkeypatch.setenv("CAT_GEMM_TILE_N", str(tile_n))
    monkeypatch.setenv("CAT_GEMM_TILE_M", str(tile_m))
    inp = rng_inputs(19, B, N, D, H, dtype)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    O = cat.cat_forward_1d(plan, to_dev(inp.X, dtype), to_dev(inp.W_A, dtype), to_dev(inp.W_V, dtype))
    import torch
    torch.cuda.synchronize()
    assert_parity(to_np(O), oracle.cat_forward_1d(inp.X, inp.W_A, inp.W_V)["O"], dtype, "O")


def _extended_line(zs, L):
    """The length-L circle the spectrum lives on: softmax values periodically
    extended (p < N: z*[p]; p > L - N: z*[p - L + N]; zero between)."""
    B, H, N = zs.shape
    out = np.zeros((B, H, L))
    out[..., :N] = zs
    if L > N:
        out[..., L - N + 1:] = zs[..., 1:]
    return out


@pytest.mark.parametrize("N", [1, 2, 3, 5, 16, 64, 197, 256, 1000, 1024, 2047, 4096])
def test_spectrum_1d(cat, N):
    say("spectrum_1d", N)
    import torch
    B, H = 2, 3
    D = 8 * H
    plan = cat.cat_plan_create("1d", "f32", B, N, D, H)
    L, L1, L2 = plan.geometry()
    logits = np.random.default_rng(N).standard_normal((B, H, N)).astype(np.float32) * 2
    probs, spec = cat.cat_step_spectrum(plan, torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    zs = oracle.softmax(logits)
    assert_parity(to_np(probs), zs, "f32", "softmax")
    ref = np.fft.fft(_extended_line(zs, L), axis=-1) / L
    got = spec.cpu().numpy()
    assert np.iscomplexobj(got) and got.shape == ref.shape
    assert_spectrum_parity(got, ref, "spectrum")


@pytest.mark.parametrize("B,N,D,H,dtype", [(1, 1, 16, 2, "f32"), (2, 2, 16, 2, "f32"), (2, 3, 16, 2, "f32"),
                                           (1, 64, 64, 4, "f32"), (2, 197, 64, 2, "f32"), (2, 197, 64, 2, "bf16"),
                                           (1, 1024, 128, 2, "bf16"), (1, 1000, 64, 4, "f32"),
                                           (1, 2048, 32, 1, "f32"), (1, 4096, 32, 2, "f32"), (1, 2047, 16, 1, "f32"),
                                           (3, 256, 96, 3, "f32"), (2, 512, 64, 32, "bf16")])
def test_mix_1d(cat, B, N, D, H, dtype):
    say("mix_1d", B, N, D, H, dtype)
    import torch
    rng = np.random.default_rng(N * 7 + D)
    logits = (rng.standard_normal((B, H, N)) * 2).astype(np.float32)
    V = rng.standard_normal((B, N, D)).astype(np.float32)
    if dtype == "bf16":
        V = W.bf16_bits_to_f32(W.round_bf16_bits(V)).reshape(V.shape)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    O = cat.cat_step_mix(plan, torch.from_numpy(logits).cuda(), to_dev(V, dtype))
    torch.cuda.synchronize()
    ref = oracle.circulant_1d(oracle.softmax(logits), V)
    assert_parity(to_np(O), ref, dtype, "O")


@pytest.mark.parametrize("conv", ["auto", "valu"])
@pytest.mark.parametrize("B,N,D,H,vscale,lscale", [(2, 1024, 128, 2, 1.0, 2.0), (1, 1024, 96, 3, 1.0, 0.0),
                                                   (2, 300, 64, 1, 1.0, 2.0), (1, 511, 96, 1, 1.0, 3.0),
                                                   (3, 257, 64, 2, 1.0, 2.0), (1, 1024, 64, 1, 1e-4, 2.0),
                                                   (1, 1024, 64, 1, 3e4, 2.0), (1, 1024, 64, 1, 1.0, 40.0),
                                                   (2, 1024, 48, 3, 1.0, 2.0)])
def test_mix_1d_l1024(cat, monkeypatch, conv, B, N, D, H, vscale, lscale):
    """The 1D conv at transform length 1024 (N = 1024, or N in 257..511 on
    the exact 2N-1 circle): bf16 storage takes the matrix-core path by
    default; CAT_CONV=valu forces the vector path on the same inputs.  Cases
    span value scales far from 1 (the fp16 stages scale each line), uniform
    scores (lscale 0) and a near one-hot softmax (lscale 40)."""
    say("mix_1d_l1024", conv, B, N, D, H, vscale, lscale)
    import torch
    if conv == "valu":
        monkeypatch.setenv("CAT_CONV", "valu")
    rng = np.random.default_rng(N * 11 + D)
    logits = (rng.standard_normal((B, H, N)) * lscale).astype(np.float32)
    V = (rng.standard_normal((B, N, D)) * vscale).astype(np.float32)
    V = W.bf16_bits_to_f32(W.round_bf16_bits(V)).reshape(V.shape)
    plan = cat.cat_plan_create("1d", "bf16", B, N, D, H)
    O = cat.cat_step_mix(plan, torch.from_numpy(logits).cuda(), to_dev(V, "bf16"))
    torch.cuda.synchronize()
    ref = oracle.circulant_1d(oracle.softmax(logits), V)
    assert_parity(to_np(O), ref, "bf16", "O")


@pytest.mark.parametrize("conv", ["auto", "fft"])
@pytest.mark.parametrize("B,N,D,H,dtype,vscale,lscale", [
    (2, 1, 64, 2, "f32", 1.0, 2.0), (2, 2, 64, 2, "bf16", 1.0, 2.0), (1, 17, 96, 1, "f32", 1.0, 2.0),
    (2, 31, 64, 1, "bf16", 1.0, 2.0), (1, 32, 64, 2, "f32", 1.0, 2.0), (2, 33, 128, 2, "bf16", 1.0, 2.0),
    (3, 100, 192, 2, "f32", 1.0, 2.0), (2, 197, 128, 2, "bf16", 1.0, 3.0), (1, 255, 64, 1, "f32", 1.0, 2.0),
    (2, 256, 256, 4, "bf16", 1.0, 2.0), (1, 256, 64, 2, "f32", 1e-4, 2.0), (1, 256, 64, 2, "bf16", 3e4, 2.0),
    (1, 200, 64, 1, "f32", 1.0, 0.0), (1, 200, 64, 1, "bf16", 1.0, 40.0), (2, 256, 96, 1, "f32", 1.0, 40.0)])
def test_mix_1d_direct(cat, monkeypatch, conv, B, N, D, H, dtype, vscale, lscale):
    """bf16 storage with N <= 256 and d a multiple of 32 takes the direct
    circulant product on the matrix cores (fp32 storage keeps the FFT path);
    CAT_CONV=fft forces the FFT path on the same inputs.
    Cases cover N = 1, lengths around the 16/32 padding steps, N = 256,
    value scales far from 1, uniform scores (lscale 0) and a near one-hot
    softmax (lscale 40)."""
    say("mix_1d_direct", conv, B, N, D, H, dtype, vscale, lscale)
    import torch
    if conv == "fft":
        monkeypatch.setenv("CAT_CONV", "fft")
    rng = np.random.default_rng(N * 13 + D)
    logits = (rng.standard_normal((B, H, N)) * lscale).astype(np.float32)
    V = (rng.standard_normal((B, N, D)) * vscale).astype(np.float32)
    if dtype == "bf16":
        V = W.bf16_bits_to_f32(W.round_bf16_bits(V)).reshape(V.shape)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    assert plan.conv_path() == ("direct" if conv == "auto" and dtype == "bf16" else "fft_valu")
    O = cat.cat_step_mix(plan, torch.from_numpy(logits).cuda(), to_dev(V, dtype))
    torch.cuda.synchronize()
    ref = oracle.circulant_1d(oracle.softmax(logits), V)
    assert_parity(to_np(O), ref, dtype, "O")


@pytest.mark.parametrize("N,D,H,dtype,path", [
    (256, 1024, 16, "bf16", "direct"), (197, 384, 6, "f32", "fft_valu"), (197, 384, 6, "bf16", "direct"),
    (64, 64, 4, "f32", "fft_valu"), (256, 64, 2, "f32", "fft_valu"),
    (257, 64, 1, "bf16", "fft_matrix"), (1024, 768, 12, "bf16", "fft_matrix"), (1024, 768, 12, "f32", "fft_valu"),
    (256, 96, 2, "f32", "fft_valu"), (128, 64, 1, "bf16", "direct"), (8192, 64, 2, "bf16", "fft_multipass"),
    (65536, 16, 1, "f32", "fft_multipass"), (2047, 64, 1, "f32", "fft_valu"), (4096, 64, 1, "bf16", "fft_valu"),
    (2049, 64, 1, "f32", "fft_multipass"), (32767, 16, 1, "bf16", "fft_multipass")])
def test_conv_path_choice(cat, N, D, H, dtype, path):
    """Which circulant-mixing path a 1D plan takes (direct: bf16, N <= 256 and
    d a multiple of 32; matrix-core FFT: transform length 1024 in bf16)."""
    say("conv_path", N, D, H, dtype, path)
    plan = cat.cat_plan_create("1d", dtype, 1, N, D, H)
    assert plan.conv_path() == path


@pytest.mark.parametrize("B,N,D,H,dtype,lscale", [
    (1, 8192, 8, 2, "f32", 2.0), (1, 8192, 8, 2, "bf16", 2.0), (2, 16384, 24, 3, "f32", 3.0),
    (1, 16384, 8, 1, "f32", 0.0), (1, 16384, 8, 1, "bf16", 40.0), (1, 32768, 8, 1, "f32", 2.0),
    (1, 65536, 8, 2, "f32", 2.0), (1, 65536, 8, 1, "bf16", 2.0), (1, 65536, 16, 1, "bf16", 40.0),
    (1, 65536, 32, 2, "bf16", 0.0), (1, 65536, 24, 4, "bf16", 2.0), (1, 65536, 8, 2, "bf16", 2.0),
    (1, 8192, 24, 4, "f32", 2.0), (2, 8192, 24, 2, "bf16", 2.0)])
def test_mix_1d_long(cat, B, N, D, H, dtype, lscale):
    """Power-of-two N beyond one workgroup's line: column, row and inverse
    column passes over HBM.  Cases span N = 2^13 .. 2^16 (square and 2:1
    splits), uniform scores (lscale 0), a near one-hot softmax (lscale 40),
    and pair blocks of 1, 2, 4 and 8 channel pairs (d = 6, 12, 8, 16); at
    N = 2^16 with bf16 storage the passes keep bf16-pair intermediates and
    the column passes take 16, 8, 4 or 2 columns a workgroup; beyond
    16384 x 16384 x 24 multiply-adds the oracle checks 1024 sampled rows."""
    say("mix_1d_long", B, N, D, H, dtype, lscale)
    import torch
    rng = np.random.default_rng(N + 5 * D)
    logits = (rng.standard_normal((B, H, N)) * lscale).astype(np.float32)
    V = rng.standard_normal((B, N, D)).astype(np.float32)
    if dtype == "bf16":
        V = W.bf16_bits_to_f32(W.round_bf16_bits(V)).reshape(V.shape)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    assert plan.conv_path() == "fft_multipass"
    O = to_np(cat.cat_step_mix(plan, torch.from_numpy(logits).cuda(), to_dev(V, dtype)))
    zs = oracle.softmax(logits)
    if N * N * D * B <= 16384 * 16384 * 24:
        assert_parity(O, oracle.circulant_1d(zs, V), dtype, "O")
    else:
        rows = np.unique(np.random.default_rng(1).integers(0, B * N, 1024))
        ref = oracle.circulant_1d(zs, V, rows=rows)
        assert_parity(O.reshape(B * N, D)[rows], ref, dtype, "O rows")


@pytest.mark.parametrize("B,N,D,H,dtype,lscale,L", [
    (1, 2049, 24, 4, "f32", 2.0, 8192), (1, 3000, 8, 2, "bf16", 2.0, 8192), (2, 4099, 8, 1, "f32", 3.0, 16384),
    (2, 5000, 24, 3, "f32", 3.0, 16384), (1, 12289, 8, 1, "bf16", 40.0, 32768), (1, 10000, 16, 2, "f32", 0.0, 32768),
    (1, 20000, 16, 2, "bf16", 2.0, 65536), (1, 32767, 8, 1, "f32", 2.0, 65536)])
def test_mix_1d_long_wrapped(cat, B, N, D, H, dtype, lscale, L):
    """Non-power-of-two N beyond 2048: the three passes on the power-of-two
    circle L >= 2N - 1 (values zero-padded, softmax line wrapped, outputs
    past N dropped).  Cases: the smallest such N (2049), a prime (4099),
    splits 128 x 64 .. 256 x 256 of L, a ragged last softmax chunk
    everywhere, uniform and near one-hot scores, pair blocks of 1, 2, 4;
    beyond 16384 x 16384 x 24 multiply-adds, 1024 sampled rows."""
    say("mix_1d_long_wrapped", B, N, D, H, dtype, lscale)
    import torch
    rng = np.random.default_rng(N + 7 * D)
    logits = (rng.standard_normal((B, H, N)) * lscale).astype(np.float32)
    V = rng.standard_normal((B, N, D)).astype(np.float32)
    if dtype == "bf16":
        V = W.bf16_bits_to_f32(W.round_bf16_bits(V)).reshape(V.shape)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    assert plan.conv_path() == "fft_multipass"
    assert plan.geometry()[0] == L
    O = to_np(cat.cat_step_mix(plan, torch.from_numpy(logits).cuda(), to_dev(V, dtype)))
    assert O.shape == (B, N, D)
    zs = oracle.softmax(logits)
    if N * N * D * B <= 16384 * 16384 * 24:
        assert_parity(O, oracle.circulant_1d(zs, V), dtype, "O")
    else:
        rows = np.unique(np.concatenate([np.random.default_rng(3).integers(0, B * N, 1024), [0, N - 1]]))
        ref = oracle.circulant_1d(zs, V, rows=rows)
        assert_parity(O.reshape(B * N, D)[rows], ref, dtype, "O rows")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16384, 6000])
def test_forward_1d_long(cat, dtype, N):
    """The whole 1D path at N = 16384 and at N = 6000 (on a circle of
    16384): projection, then the three-pass mixing, on 512 sampled rows."""
    B, D, H = 1, 64, 2
    say("forward_1d_long", B, N, D, H, dtype)
    import torch
    inp = rng_inputs(23, B, N, D, H, dtype)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    assert plan.conv_path() == "fft_multipass"
    O = cat.cat_forward_1d(plan, to_dev(inp.X, dtype), to_dev(inp.W_A, dtype), to_dev(inp.W_V, dtype))
    torch.cuda.synchronize()
    rows = np.unique(np.random.default_rng(2).integers(0, B * N, 512))
    ref = oracle.cat_forward_1d(inp.X, inp.W_A, inp.W_V, rows=rows)["O"]
    assert_parity(to_np(O).reshape(B * N, D)[rows], ref, dtype, "O rows")


# ------------------------------------------------------------------ 1D mixing backward
@pytest.mark.parametrize("B,N,D,H,dtype,path", [
    (2, 64, 64, 4, "f32", "fft_valu"), (1, 1, 16, 2, "f32", "fft_valu"), (2, 2, 16, 2, "f32", "fft_valu"),
    (1, 197, 96, 3, "f32", "fft_valu"), (3, 2047, 16, 1, "f32", "fft_valu"), (1, 1000, 64, 4, "f32", "fft_valu"),
    (1, 4096, 32, 2, "f32", "fft_valu"), (2, 1024, 128, 2, "bf16", "fft_matrix"), (2, 128, 64, 1, "bf16", "direct"),
    (1, 197, 384, 6, "bf16", "direct"), (2, 512, 64, 32, "bf16", "fft_valu")])
def test_mix_backward_1d(cat, B, N, D, H, dtype, path):
    """Gradients of the mixing for an output gradient dO: dV on the plan's
    own mixing path (reversed logits), dlogits from the FFT cross-correlation
    and the softmax Jacobian, against the oracle's direct sums.  Covers
    N = 1 and 2, primes and other N on the 2N - 1 circle, L up to 4096 and
    every 1D mixing path for dV.  dlogits is computed in fp32 from the stored
    values, so it meets the fp32 bar in both storage dtypes."""
    say("mix_backward_1d", B, N, D, H, dtype, path)
    import torch
    rng = np.random.default_rng(N * 3 + D)
    logits = (rng.standard_normal((B, H, N)) * 2).astype(np.float32)
    V = rng.standard_normal((B, N, D)).astype(np.float32)
    dO = rng.standard_normal((B, N, D)).astype(np.float32)
    if dtype == "bf16":
        V = W.bf16_bits_to_f32(W.round_bf16_bits(V)).reshape(V.shape)
        dO = W.bf16_bits_to_f32(W.round_bf16_bits(dO)).reshape(dO.shape)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    assert plan.conv_path() == path
    dlogits, dV = cat.cat_step_mix_backward_1d(plan, torch.from_numpy(logits).cuda(), to_dev(V, dtype),
                                               to_dev(dO, dtype))
    torch.cuda.synchronize()
    ref = oracle.mix_backward_1d(logits, V, dO)
    assert_parity(to_np(dV), ref["dV"], dtype, "dV")
    got = to_np(dlogits)
    assert_parity(got, ref["dz"], "f32", "dlogits")
    # each line sums to zero, up to fp32 rounding of its entries
    assert np.all(np.abs(got.sum(axis=-1)) <= 1e-5 * np.abs(got).sum(axis=-1) + 1e-7)


def test_mix_backward_1d_workload_full_size(cat):
    """The mixing backward at the benchmarked shape (B = 16, N = 1024, D = 768,
    H = 12, bf16; V and the logits from the workload's projection, dO seeded),
    on the launch configuration bench.py --backward times; the oracle checks
    the first and the last sequence in full."""
    import torch
    wl = W.WORKLOADS["cat1d_gpt2_n1024"]
    say("mix_backward_full", wl.name)
    inp = W.make_inputs(wl)
    plan = cat.cat_plan_create("1d", wl.dtype, wl.B, wl.N, wl.D, wl.H)
    V, z = cat.cat_step_project(plan, to_dev(inp.X, wl.dtype), to_dev(inp.W_A, wl.dtype), to_dev(inp.W_V, wl.dtype))
    g = np.random.default_rng(99).standard_normal((wl.B, wl.N, wl.D)).astype(np.float32)
    g = W.bf16_bits_to_f32(W.round_bf16_bits(g)).reshape(g.shape)
    dlogits, dV = cat.cat_step_mix_backward_1d(plan, z, V, to_dev(g, wl.dtype))
    torch.cuda.synchronize()
    zc, Vc, dz, dVc = to_np(z), to_np(V), to_np(dlogits), to_np(dV)
    for b in (0, wl.B - 1):
        ref = oracle.mix_backward_1d(zc[b:b + 1], Vc[b:b + 1], g[b:b + 1])
        assert_parity(dVc[b:b + 1], ref["dV"], wl.dtype, f"dV b={b}")
        assert_parity(dz[b:b + 1], ref["dz"], "f32", f"dlogits b={b}")


@pytest.mark.parametrize("B,N,D,H,dtype,path", [
    (2, 64, 64, 4, "f32", "fft_valu"), (1, 128, 128, 2, "bf16", "direct"), (2, 1024, 128, 2, "bf16", "fft_matrix"),
    (1, 200, 96, 3, "f32", "fft_valu"), (4, 6, 16, 2, "f32", "fft_valu"), (1, 8, 64, 32, "bf16", "fft_valu"),
    (2, 512, 96, 12, "bf16", "fft_valu"), (8, 1000, 64, 4, "f32", "fft_valu"), (2, 4096, 32, 2, "f32", "fft_valu"),
    (1, 197, 64, 2, "f32", "fft_valu"), (3, 61, 48, 3, "bf16", "fft_valu"), (1, 1, 16, 2, "f32", "fft_valu"),
    (1, 8192, 32, 2, "f32", "fft_multipass"), (1, 3000, 16, 1, "bf16", "fft_multipass")])
def test_backward_1d(cat, B, N, D, H, dtype, path):
    """Gradients of the whole 1D forward (dX, dW_A, dW_V) against the oracle's
    chain rule; the mixing runs on the plan's path, the products on the
    projection GEMM.  B N = 197, 183 and 1 are not multiples of 8: X^T rows
    are padded with zeros to 16-byte multiples; N = 8192 and 3000 run the
    three-pass path (L = N, and L = 8192 >= 2N - 1)."""
    say("backward_1d", B, N, D, H, dtype, path)
    import torch
    inp = rng_inputs(31, B, N, D, H, dtype)
    g = np.random.default_rng(N + D).standard_normal((B, N, D)).astype(np.float32)
    if dtype == "bf16":
        g = W.bf16_bits_to_f32(W.round_bf16_bits(g)).reshape(g.shape)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    assert plan.conv_path() == path
    dX, dWA, dWV = cat.cat_backward_1d(plan, to_dev(inp.X, dtype), to_dev(inp.W_A, dtype), to_dev(inp.W_V, dtype),
                                       to_dev(g, dtype))
    torch.cuda.synchronize()
    ref = oracle.cat_backward_1d(inp.X, inp.W_A, inp.W_V, g)
    assert_parity(to_np(dX), ref["dX"], dtype, "dX")
    check_weight_grads(ref, inp.X, {"dW_A": dWA, "dW_V": dWV}, dtype)


def check_weight_grads(ref, X, got, dtype):
    """dW_V = X^T dV and dW_A = X^T dz^T sum over K = B N tokens.  The
    relative L2 bar is the stated one; the fp32 max-abs bar is derived from
    fp32 accumulation over K terms and the fp32 bar of the mixing step that
    makes dV and dz (helpers.sum_bar), since the stated 1e-4 is for
    unit-scale outputs of short sums."""
    B, N, _ = X.shape
    K = B * N
    rms_x = float(np.sqrt(np.mean(np.asarray(X, np.float64) ** 2)))
    for name, fac in (("dW_A", "dz"), ("dW_V", "dV")):
        g, r = to_np(got[name]), ref[name]
        rl = rel_l2(g, r)
        assert rl <= (1e-5 if dtype == "f32" else 2e-2), f"{name}: rel_l2={rl:.3e}"
        if dtype == "f32":
            bar = sum_bar(K, rms_x, float(np.sqrt(np.mean(ref[fac] ** 2))))
            m = float(np.max(np.abs(g - r)))
            assert m <= bar, f"{name}: max_abs={m:.3e} > bar {bar:.3e} (K={K})"


def test_backward_1d_empty_batch(cat):
    """B = 0: the weight gradients are empty sums, written as zeros."""
    import torch
    for dtype in ("f32", "bf16"):
        plan = cat.cat_plan_create("1d", dtype, 0, 64, 32, 2)
        dt = torch.float32 if dtype == "f32" else torch.bfloat16
        X = torch.empty((0, 64, 32), dtype=dt, device="cuda")
        dX, dWA, dWV = cat.cat_backward_1d(plan, X, torch.ones((32, 2), dtype=dt, device="cuda"),
                                           torch.ones((32, 32), dtype=dt, device="cuda"), X,
                                           workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert dX.shape == (0, 64, 32)
        assert torch.count_nonzero(dWA).item() == 0 and torch.count_nonzero(dWV).item() == 0


@pytest.mark.parametrize("B,N,D,H,dtype", [(1, 8192, 16, 2, "f32"), (2, 5000, 16, 2, "bf16"), (1, 2500, 32, 1, "f32"),
                                           (1, 16384, 8, 1, "bf16")])
def test_mix_backward_1d_long(cat, B, N, D, H, dtype):
    """The mixing backward on the three-pass path: dV as the forward mixing
    with reversed logits, dlogits from the cross-correlation spectra of every
    pair of a head summed before one inverse transform (L = N for N = 8192
    and 16384; on the L >= 2N - 1 circle, folded onto mod-N lags, for 5000
    and 2500), against the oracle's direct sums."""
    say("mix_backward_long", B, N, D, H, dtype)
    import torch
    rng = np.random.default_rng(N + 7 * D)
    logits = (rng.standard_normal((B, H, N)) * 2).astype(np.float32)
    V = rng.standard_normal((B, N, D)).astype(np.float32)
    dO = rng.standard_normal((B, N, D)).astype(np.float32)
    if dtype == "bf16":
        V = W.bf16_bits_to_f32(W.round_bf16_bits(V)).reshape(V.shape)
        dO = W.bf16_bits_to_f32(W.round_bf16_bits(dO)).reshape(dO.shape)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    assert plan.conv_path() == "fft_multipass"
    dlogits, dV = cat.cat_step_mix_backward_1d(plan, torch.from_numpy(logits).cuda(), to_dev(V, dtype),
                                               to_dev(dO, dtype))
    torch.cuda.synchronize()
    ref = oracle.mix_backward_1d(logits, V, dO)
    assert_parity(to_np(dV), ref["dV"], dtype, "dV")
    got = to_np(dlogits)
    assert_parity(got, ref["dz"], "f32", "dlogits")
    assert np.all(np.abs(got.sum(axis=-1)) <= 1e-5 * np.abs(got).sum(axis=-1) + 1e-7)


def test_mix_backward_1d_rejections(cat):
    """2D plans are the wrong kind for the 1D mixing backward."""
    import torch
    p2 = cat.cat_plan_create("2d", "f32", 1, 64, 16, 2, Hg=8, Wg=8)
    with pytest.raises(cat.CatError) as e:
        cat.cat_step_mix_backward_1d(p2, torch.zeros((1, 2, 64), device="cuda"), torch.zeros((1, 64, 16), device="cuda"),
                                     torch.zeros((1, 64, 16), device="cuda"))
    assert e.value.status == -5


# ------------------------------------------------------------------ 1D forward
@pytest.mark.parametrize("B,N,D,H,dtype", [(1, 64, 64, 4, "f32"), (2, 37, 48, 3, "f32"), (3, 100, 64, 4, "bf16"),
                                           (1, 1, 32, 2, "f32"), (2, 197, 96, 3, "f32"), (1, 1024, 64, 1, "bf16"),
                                           (5, 128, 72, 9, "f32"), (2, 64, 128, 32, "bf16")])
def test_forward_1d_small(cat, B, N, D, H, dtype):
    say("forward_1d", B, N, D, H, dtype)
    import torch
    inp = rng_inputs(5, B, N, D, H, dtype)
    plan = cat.cat_plan_create("1d", dtype, B, N, D, H)
    O = cat.cat_forward_1d(plan, to_dev(inp.X, dtype), to_dev(inp.W_A, dtype), to_dev(inp.W_V, dtype))
    torch.cuda.synchronize()
    ref = oracle.cat_forward_1d(inp.X, inp.W_A, inp.W_V)["O"]
    assert_parity(to_np(O), ref, dtype, "O")


WL1D = [n for n, w in W.WORKLOADS.items() if w.kind == "1d"]


@pytest.mark.parametrize("name", WL1D)
def test_forward_1d_workload_full_size(cat, name):
    """The workload at its full size, in the launch configuration bench.py
    times; the oracle recomputes a sample of whole images."""
    wl = W.WORKLOADS[name]
    say("forward_1d_workload", name)
    import torch
    inp = W.make_inputs(wl)
    plan = cat.cat_plan_create("1d", wl.dtype, wl.B, wl.N, wl.D, wl.H)
    O = cat.cat_forward_1d(plan, to_dev(inp.X, wl.dtype), to_dev(inp.W_A, wl.dtype), to_dev(inp.W_V, wl.dtype))
    torch.cuda.synchronize()
    O = to_np(O)
    assert np.all(np.isfinite(O))
    if wl.N > 4096:  # long sequence: 256 sampled rows of the one sequence
        rows = np.unique(np.random.default_rng(3).integers(0, wl.N, 256))
        ref = oracle.cat_forward_1d(inp.X[:1], inp.W_A, inp.W_V, rows=rows)["O"]
        assert_parity(O[0][rows], ref, wl.dtype, f"{name} rows")
        return
    for b in sorted({0, wl.B // 2, wl.B - 1}):
        ref = oracle.cat_forward_1d(inp.X[b:b + 1], inp.W_A, inp.W_V)["O"][0]
        assert_parity(O[b], ref, wl.dtype, f"{name} b={b}")


def test_prime_length_is_exactly_circular(cat):
    """N = 197 must wrap mod 197: the GPU result matches the oracle and is far
    from what a length-256 zero-padded circular product would give."""
    say("prime_length")
    import torch
    B, N, D, H = 2, 197, 64, 2
    rng = np.random.default_rng(197)
    logits = (rng.standard_normal((B, H, N)) * 3).astype(np.float32)
    V = rng.standard_normal((B, N, D)).astype(np.float32)
    plan = cat.cat_plan_create("1d", "f32", B, N, D, H)
    O = to_np(cat.cat_step_mix(plan, torch.from_numpy(logits).cuda(), to_dev(V, "f32")))
    zs = oracle.softmax(logits)
    assert_parity(O, oracle.circulant_1d(zs, V), "f32", "O")
    wrong = np.zeros_like(O)
    for h in range(H):
        w = np.zeros((B, 256))
        w[:, :N] = zs[:, h]
        v = np.zeros((B, 256, D // H))
        v[:, :N] = V[:, :, h * (D // H):(h + 1) * (D // H)]
        wrong[:, :, h * (D // H):(h + 1) * (D // H)] = np.fft.ifft(
            np.fft.fft(w, axis=1)[:, :, None] * np.fft.fft(v, axis=1), axis=1).real[:, :N]
    assert rel_l2(O, wrong) > 1e-2


def test_determinism_1d(cat):
    say("determinism_1d")
    import torch
    wl = W.WORKLOADS[W.HEADLINE].with_(B=2)
    inp = W.make_inputs(wl, batch=2)
    plan = cat.cat_plan_create("1d", wl.dtype, 2, wl.N, wl.D, wl.H)
    args = [to_dev(a, wl.dtype) for a in (inp.X, inp.W_A, inp.W_V)]
    O1 = cat.cat_forward_1d(plan, *args)
    O2 = cat.cat_forward_1d(plan, *args)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)


# ------------------------------------------------------------------ 2D
GRIDS = [(1, 1), (2, 3), (3, 4), (4, 4), (6, 8), (8, 8), (12, 12), (16, 16)]
# patch grids of common vision-transformer resolutions (7 = a radix-7 DFT)
VIT_GRIDS = [(7, 7), (14, 14), (24, 24), (28, 28), (48, 48)]


@pytest.mark.parametrize("Hg,Wg", GRIDS + VIT_GRIDS + [(32, 32), (96, 96)])
def test_scores_2d(cat, Hg, Wg):
    say("scores_2d", Hg, Wg)
    import torch
    B, D, H = (1 if Hg * Wg > 4096 else 2), 16, 2
    rng = np.random.default_rng(Hg * 100 + Wg)
    Q = (rng.standard_normal((B, Hg * Wg, D)) * 0.5).astype(np.float32)
    K = (rng.standard_normal((B, Hg * Wg, D)) * 0.5).astype(np.float32)
    plan = cat.cat_plan_create("2d", "f32", B, Hg * Wg, D, H, Hg, Wg)
    probs = to_np(cat.cat_step_scores_2d(plan, torch.from_numpy(Q).cuda(), torch.from_numpy(K).cuda()))
    a = oracle.scores_bccb_2d(Q, K, Hg, Wg, H)
    ref = oracle.softmax(a.reshape(B, H, -1))
    assert_parity(probs, ref, "f32", "a*")


@pytest.mark.parametrize("B,D,H", [(1, 24, 4), (1, 40, 4), (1, 8, 4), (1, 64, 1), (3, 64, 1), (1, 48, 3)])
def test_scores_2d_96_pair_groups(cat, B, D, H):
    """The 96 x 96 score kernel takes a head's channel pairs two to a
    workgroup: d = 6 and 10 (3 and 5 pairs) leave a last group of one pair,
    d = 2 a head of one pair; d = 64 is the workload's 32 pairs, for one and
    three heads; d = 16 gives 8 pairs for each of three heads."""
    say("scores_2d_96_groups", B, D, H)
    import torch
    G = 96
    rng = np.random.default_rng(D * 10 + H)
    Q = (rng.standard_normal((B, G * G, D)) * 0.5).astype(np.float32)
    K = (rng.standard_normal((B, G * G, D)) * 0.5).astype(np.float32)
    plan = cat.cat_plan_create("2d", "f32", B, G * G, D, H, G, G)
    probs = to_np(cat.cat_step_scores_2d(plan, torch.from_numpy(Q).cuda(), torch.from_numpy(K).cuda()))
    a = oracle.scores_bccb_2d(Q, K, G, G, H)
    ref = oracle.softmax(a.reshape(B, H, -1))
    assert_parity(probs, ref, "f32", "a*")


@pytest.mark.parametrize("Hg,Wg,dtype", [(g[0], g[1], "f32") for g in GRIDS + VIT_GRIDS] +
                         [(12, 12, "bf16"), (14, 14, "bf16"), (24, 24, "bf16"), (32, 32, "f32"), (32, 32, "bf16"),
                          (96, 96, "f32"), (96, 96, "bf16")])
def test_mix_2d(cat, Hg, Wg, dtype):
    say("mix_2d", Hg, Wg, dtype)
    import torch
    B, D, H = (1 if Hg * Wg > 4096 else 2), 16, 2
    N = Hg * Wg
    rng = np.random.default_rng(N + 3)
    logits = (rng.standard_normal((B, H, N)) * 2).astype(np.float32)
    V = rng.standard_normal((B, N, D)).astype(np.float32)
    if dtype == "bf16":
        V = W.bf16_bits_to_f32(W.round_bf16_bits(V)).reshape(V.shape)
    plan = cat.cat_plan_create("2d", dtype, B, N, D, H, Hg, Wg)
    O = to_np(cat.cat_step_mix(plan, torch.from_numpy(logits).cuda(), to_dev(V, dtype)))
    ref = oracle.bccb_2d(oracle.softmax(logits).reshape(B, H, Hg, Wg), V)
    assert_parity(O, ref, dtype, "O")


@pytest.mark.parametrize("G", [32, 96])
@pytest.mark.parametrize("case", ["normal", "uniform", "onehot", "tiny", "huge"])
def test_mix_2d_matrix(cat, G, case):
    """The 2D mixing on the matrix cores (bf16, square grids of 32 and 96):
    ordinary logits, uniform logits (the filter is a constant: every output
    is the grid mean), a near one-hot filter (a cyclic shift of the grid),
    and value scales 1e-4 and 3e4 (the per-grid power-of-two scaling)."""
    say("mix_2d_matrix", G, case)
    import torch
    B, D, H = (1, 64, 2) if G == 96 else (2, 64, 2)
    N = G * G
    rng = np.random.default_rng(G + len(case))
    logits = (rng.standard_normal((B, H, N)) * 2).astype(np.float32)
    if case == "uniform":
        logits[:] = 0.25
    elif case == "onehot":
        logits[:, :, 5 * G + 7] = 40.0
    vs = {"tiny": 1e-4, "huge": 3e4}.get(case, 1.0)
    V = (rng.standard_normal((B, N, D)) * vs).astype(np.float32)
    V = W.bf16_bits_to_f32(W.round_bf16_bits(V)).reshape(V.shape)
    plan = cat.cat_plan_create("2d", "bf16", B, N, D, H, G, G)
    assert plan.conv_path() == "fft_matrix"
    O = to_np(cat.cat_step_mix(plan, torch.from_numpy(logits).cuda(), to_dev(V, "bf16")))
    ref = oracle.bccb_2d(oracle.softmax(logits).reshape(B, H, G, G), V)
    assert_parity(O, ref, "bf16", "O")


@pytest.mark.parametrize("B,Hg,Wg,D,H,dtype,ss", [(1, 3, 4, 16, 2, "f32", 1.0), (2, 8, 8, 32, 2, "f32", 0.3),
                                                  (2, 12, 12, 48, 3, "bf16", 0.3), (1, 6, 8, 64, 1, "f32", 1.0),
                                                  (2, 16, 16, 64, 4, "bf16", 0.2), (2, 8, 8, 24, 4, "f32", 0.5),
                                                  (1, 12, 12, 24, 2, "bf16", 0.3), (2, 32, 32, 64, 2, "bf16", 0.3),
                                                  (2, 14, 14, 64, 2, "bf16", 0.3), (1, 7, 7, 32, 2, "f32", 0.5),
                                                  (1, 24, 24, 64, 2, "bf16", 0.3), (1, 28, 28, 32, 2, "f32", 0.3),
                                                  (1, 48, 48, 64, 2, "bf16", 0.2), (1, 96, 96, 16, 2, "f32", 0.3),
                                                  (1, 96, 96, 16, 2, "bf16", 0.3)])
def test_forward_2d_small(cat, B, Hg, Wg, D, H, dtype, ss):
    say("forward_2d", B, Hg, Wg, D, H, dtype, ss)
    import torch
    inp = rng_inputs_2d(9, B, Hg, Wg, D, H, dtype, score_scale=ss)
    plan = cat.cat_plan_create("2d", dtype, B, Hg * Wg, D, H, Hg, Wg)
    O = cat.cat_forward_bccb_2d(plan, *[to_dev(a, dtype) for a in (inp.X, inp.W_Q, inp.W_K, inp.W_V)])
    torch.cuda.synchronize()
    ref = oracle.cat_forward_bccb_2d(inp.X, inp.W_Q, inp.W_K, inp.W_V, Hg, Wg, H)["O"]
    assert_parity(to_np(O), ref, dtype, "O")


@pytest.mark.parametrize("B,Hg,Wg,D,H,dtype", [
    (2, 8, 8, 64, 4, "f32"), (1, 12, 12, 48, 3, "bf16"), (2, 2, 3, 16, 2, "f32"), (1, 16, 16, 32, 2, "bf16"),
    (1, 6, 8, 24, 2, "f32"), (1, 1, 1, 16, 2, "f32"), (1, 32, 32, 64, 2, "f32"), (1, 96, 96, 64, 2, "bf16"),
    (1, 14, 14, 64, 2, "bf16"), (1, 7, 7, 32, 2, "f32")])
def test_forward_cat_2d(cat, B, Hg, Wg, D, H, dtype):
    """The CAT-scored 2D variant (X W_A scores, softmax over the grid, BCCB
    mixing) against the oracle, on grids from 1 x 1 to 96 x 96."""
    say("forward_cat_2d", B, Hg, Wg, D, H, dtype)
    import torch
    inp = rng_inputs_2d(17, B, Hg, Wg, D, H, dtype)
    W_A = (np.random.default_rng(Hg * Wg + D).standard_normal((D, H)) * 1.5 / np.sqrt(D)).astype(np.float32)
    if dtype == "bf16":
        W_A = W.bf16_bits_to_f32(W.round_bf16_bits(W_A)).reshape(W_A.shape)
    plan = cat.cat_plan_create("2d", dtype, B, Hg * Wg, D, H, Hg, Wg)
    O = cat.cat_forward_cat_2d(plan, to_dev(inp.X, dtype), to_dev(W_A, dtype), to_dev(inp.W_V, dtype))
    torch.cuda.synchronize()
    ref = oracle.cat_scored_forward_2d(inp.X, W_A, inp.W_V, Hg, Wg)["O"]
    assert_parity(to_np(O), ref, dtype, "O")


def test_forward_cat_2d_workload_full_size(cat):
    """The CAT-scored variant at the 96 x 96 workload (B = 8, D = 384, H = 6,
    bf16) as bench.py --variant cat2d runs it; the oracle recomputes two
    (image, head) slices end to end."""
    import torch
    wl = W.WORKLOADS["bccb2d_1536px_96x96"]
    say("forward_cat_2d_full", wl.name)
    inp = W.make_inputs(wl)
    W_A = (np.random.default_rng(wl.seed + 1000).standard_normal((wl.D, wl.H)) / np.sqrt(wl.D)).astype(np.float32)
    W_A = W.bf16_bits_to_f32(W.round_bf16_bits(W_A)).reshape(W_A.shape)
    plan = cat.cat_plan_create("2d", wl.dtype, wl.B, wl.N, wl.D, wl.H, wl.Hg, wl.Wg)
    O = to_np(cat.cat_forward_cat_2d(plan, to_dev(inp.X, wl.dtype), to_dev(W_A, wl.dtype), to_dev(inp.W_V, wl.dtype)))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(O))
    d = wl.d
    for b, h in [(0, 0), (wl.B - 1, wl.H - 1)]:
        hs = slice(h * d, (h + 1) * d)
        ref = oracle.cat_scored_forward_2d(inp.X[b:b + 1], W_A[:, h:h + 1], inp.W_V[:, hs], wl.Hg, wl.Wg)["O"][0]
        assert_parity(O[b][:, hs], ref, wl.dtype, f"b={b} h={h}")


def test_forward_cat_2d_rejections(cat):
    import torch
    p1 = cat.cat_plan_create("1d", "f32", 1, 64, 64, 4)
    X = torch.zeros((1, 64, 64), device="cuda")
    with pytest.raises(cat.CatError) as e:
        cat.cat_forward_cat_2d(p1, X, torch.zeros((64, 4), device="cuda"), torch.zeros((64, 64), device="cuda"))
    assert e.value.status == -5
    p2 = cat.cat_plan_create("2d", "f32", 1, 64, 128, 64, 8, 8)  # 64 heads of 2 channels
    X2 = torch.zeros((1, 64, 128), device="cuda")
    with pytest.raises(cat.CatError) as e:
        cat.cat_forward_cat_2d(p2, X2, torch.zeros((128, 64), device="cuda"), torch.zeros((128, 128), device="cuda"))
    assert e.value.status == -2


def test_forward_2d_workload_full_size(cat):
    """96x96 grid, B=8, D=384, H=6, bf16, at full size; the oracle recomputes
    two (image, head) slices end to end."""
    wl = W.WORKLOADS["bccb2d_1536px_96x96"]
    say("forward_2d_workload", wl.name)
    import torch
    inp = W.make_inputs(wl)
    plan = cat.cat_plan_create("2d", wl.dtype, wl.B, wl.N, wl.D, wl.H, wl.Hg, wl.Wg)
    O = cat.cat_forward_bccb_2d(plan, *[to_dev(a, wl.dtype) for a in (inp.X, inp.W_Q, inp.W_K, inp.W_V)])
    torch.cuda.synchronize()
    O = to_np(O)
    assert np.all(np.isfinite(O))
    d = wl.d
    for b, h in [(0, 0), (wl.B - 1, wl.H - 1)]:
        hs = slice(h * d, (h + 1) * d)
        ref = oracle.cat_forward_bccb_2d(inp.X[b:b + 1], inp.W_Q[:, hs], inp.W_K[:, hs], inp.W_V[:, hs],
                                         wl.Hg, wl.Wg, 1)["O"][0]
        assert_parity(O[b][:, hs], ref, wl.dtype, f"b={b} h={h}")


def test_determinism_2d(cat):
    say("determinism_2d")
    import torch
    inp = rng_inputs_2d(2, 2, 12, 12, 48, 3, "bf16", score_scale=0.3)
    plan = cat.cat_plan_create("2d", "bf16", 2, 144, 48, 3, 12, 12)
    args = [to_dev(a, "bf16") for a in (inp.X, inp.W_Q, inp.W_K, inp.W_V)]
    O1 = cat.cat_forward_bccb_2d(plan, *args)
    O2 = cat.cat_forward_bccb_2d(plan, *args)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)


# ------------------------------------------------------------------ errors
def test_plan_kind_mismatch_and_misalignment(cat):
    say("errors")
    import ctypes
    import torch
    plan = cat.cat_plan_create("1d", "f32", 1, 64, 64, 4)
    X = torch.zeros(1, 64, 64, device="cuda")
    Wv = torch.zeros(64, 64, device="cuda")
    ws = cat.alloc_workspace(plan)
    lib = cat.lib()
    st = lib.cat_forward_bccb_2d(ctypes.c_void_p(plan.handle), ctypes.c_void_p(X.data_ptr()),
                                 ctypes.c_void_p(Wv.data_ptr()), ctypes.c_void_p(Wv.data_ptr()),
                                 ctypes.c_void_p(Wv.data_ptr()), ctypes.c_void_p(X.data_ptr()),
                                 ctypes.c_void_p(ws.data_ptr()), None)
    assert st == -5
    flat = torch.zeros(64 * 64 + 4, device="cuda")
    st = lib.cat_forward_1d(ctypes.c_void_p(plan.handle), ctypes.c_void_p(flat.data_ptr() + 4),
                            ctypes.c_void_p(Wv.data_ptr()), ctypes.c_void_p(Wv.data_ptr()),
                            ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(ws.data_ptr()), None)
    assert st == -1
    assert "aligned" in lib.cat_last_error().decode()


def test_empty_batch_is_a_no_op(cat):
    say("empty_batch")
    import torch
    for kind, extra in [("1d", {}), ("2d", {"Hg": 8, "Wg": 8})]:
        plan = cat.cat_plan_create(kind, "f32", 0, 64, 32, 2, **extra)
        X = torch.empty(0, 64, 32, device="cuda")
        Wm = torch.zeros(32, 32, device="cuda")
        if kind == "1d":
            O = cat.cat_forward_1d(plan, X, torch.zeros(32, 2, device="cuda"), Wm)
        else:
            O = cat.cat_forward_bccb_2d(plan, X, Wm, Wm, Wm)
        torch.cuda.synchronize()
        assert O.shape == (0, 64, 32)
