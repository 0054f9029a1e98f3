#!/usr/bin/env python3
"""Throughput of the circulant softmax attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole forward pass (projection MFMA GEMM, softmax + filter
spectrum, fused FFT-convolution; in 2D also the score correlation) over one
batch of seeded synthetic input already resident in device memory.  The
default workload is CAT 1D at N=1024, D=768 (B=16, H=12, bf16 storage, fp32
compute).  Input/output/workspace buffers are rotated over enough sets to
exceed the 256 MB Infinity Cache, so every step reads its inputs from HBM.

Rank 0 prints one JSON line on stdout; progress goes to stderr.  The line
carries the headline metric, a roofline entry for the slowest kernel (its
algorithmic bytes or flops per launch over its average launch time, measured
with HIP events recorded by the library around each kernel in an
instrumented pass of the same K steps) and the fp64 CPU oracle timed on a
bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"mfma_bf16": 2500.0, "mfma_f16": 2500.0, "mfma_f32": 157.3, "valu_f32": 78.6}
MALL_BYTES = 256 << 20


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def fft_flops(L: int) -> float:
    """Conventional flop count of one complex transform of L points."""
    return 5.0 * L * math.log2(L) if L > 1 else 0.0


def kernel_model(wl, L: int, ngrp: int, fused_spectrum: bool = False, direct: bool = False,
                 multipass: bool = False):
    """Algorithmic bytes and flops of each kernel of one forward call.

    fused_spectrum: the 1D conv ran on the matrix cores and computed the
    softmax spectrum itself (no spectrum launch): it reads the logits instead
    of a spectrum, and its flops are the matrix products it executes (four
    32x32x32 complex products per line, each 4 x 2 x 32^3 real flops, plus two
    per workgroup of 16 channels for the spectrum line).

    direct: the 1D mixing ran as the direct product circ(z*) V on the matrix
    cores ("directconv", softmax included): it reads V and the logits and
    writes O; its flops are the product's 2 N^2 d per (batch, head).

    multipass: the 1D mixing ran as three passes over HBM (three launches
    each for the spectrum and for the values).  The bytes are the algorithmic
    ones (V read, O written, spectrum read; logits read, spectrum written),
    not the passes' intermediates, so hbm_frac shows what the passes cost."""
    s = 4 if wl.dtype == "f32" else 2
    B, N, D, H, d = wl.B, wl.N, wl.D, wl.H, wl.d
    T = B * N
    BH = B * H
    lines = BH * (d // 2)
    spec_bytes = BH * L * 8
    m = {}
    if wl.kind == "1d":
        # X read once, W_V and W_A, V written (storage dtype) and z written (fp32)
        m["project"] = dict(bytes=T * D * s + D * (D + H) * s + T * D * s + BH * N * 4,
                            flops=2.0 * T * D * (D + H), unit="mfma_bf16" if s == 2 else "mfma_f32")
        m["spectrum"] = dict(bytes=BH * N * 4 + spec_bytes, flops=BH * (fft_flops(L) + 4.0 * N), unit="valu_f32")
    else:
        m["project"] = dict(bytes=T * D * s + 3 * D * D * s + 2 * T * D * 4 + T * D * s,
                            flops=2.0 * T * D * 3 * D, unit="mfma_bf16" if s == 2 else "mfma_f32")
        m["scores"] = dict(bytes=2 * T * D * 4 + BH * ngrp * L * 8,
                           flops=lines * (2 * fft_flops(L) + 8.0 * L), unit="valu_f32")
        m["psum"] = dict(bytes=BH * ngrp * L * 8 + BH * L * 8, flops=2.0 * BH * (ngrp - 1) * L, unit="valu_f32")
        m["spectrum"] = dict(bytes=BH * L * 8 + spec_bytes,
                             flops=BH * (2 * fft_flops(L) + 4.0 * N), unit="valu_f32")
    m["fftconv"] = dict(bytes=2 * T * D * s + spec_bytes, flops=lines * (2 * fft_flops(L) + 6.0 * L), unit="valu_f32")
    if wl.Hg:
        # the matrix-core 2D conv: four dense G x G x G complex products per
        # channel pair (4 x 4 x 2 G^3 real flops, bf16 operands); it reads V
        # and S and writes O
        G = wl.Hg
        m["fftconv_matrix"] = dict(bytes=2 * T * D * s + spec_bytes, flops=lines * 4 * 4 * 2.0 * G ** 3,
                                   unit="mfma_bf16")
    if fused_spectrum:
        cplx = 4 * 2.0 * 32 ** 3  # one 32x32x32 complex product in real flops
        m["fftconv"] = dict(bytes=2 * T * D * s + BH * N * 4, flops=lines * 4 * cplx + B * H * (d // 16) * 2 * cplx,
                            unit="mfma_f16")
    if multipass:
        m["spectrum"] = dict(bytes=BH * N * 4 + spec_bytes, flops=BH * fft_flops(L), unit="valu_f32")
        m["fftconv"] = dict(bytes=2 * T * D * s + spec_bytes, flops=lines * (2 * fft_flops(L) + 6.0 * L),
                            unit="valu_f32")
    if direct:
        m["directconv"] = dict(bytes=2 * T * D * s + BH * N * 4, flops=2.0 * BH * N * N * d,
                               unit="mfma_bf16" if s == 2 else "mfma_f32")
    return m


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "fftconv": ["circulant_softmax_attention_amd/csrc/cat_mconv.hip",
                "circulant_softmax_attention_amd/csrc/cat_fftconv.hpp", "circulant_softmax_attention_amd/csrc/cat_fft.hpp",
                "circulant_softmax_attention_amd/csrc/cat_common.hpp"],
    "project": ["circulant_softmax_attention_amd/csrc/cat_gemm.hip", "circulant_softmax_attention_amd/csrc/cat_common.hpp"],
}
KERNEL_SOURCES["directconv"] = ["circulant_softmax_attention_amd/csrc/cat_dconv.hip",
                                 "circulant_softmax_attention_amd/csrc/cat_common.hpp"]
KERNEL_SOURCES["spectrum"] = KERNEL_SOURCES["fftconv"] + ["circulant_softmax_attention_amd/csrc/cat_score96.hip"]
KERNEL_SOURCES["scores"] = ["circulant_softmax_attention_amd/csrc/cat_score96.hip",
                            "circulant_softmax_attention_amd/csrc/cat_fftconv.hpp",
                            "circulant_softmax_attention_amd/csrc/cat_fft.hpp",
                            "circulant_softmax_attention_amd/csrc/cat_common.hpp"]
KERNEL_SOURCES["fftconv_matrix"] = ["circulant_softmax_attention_amd/csrc/cat_bconv.hip",
                                    "circulant_softmax_attention_amd/csrc/cat_common.hpp"]
KERNEL_SOURCES["score_grad"] = ["circulant_softmax_attention_amd/csrc/cat_fftconv.hpp",
                                "circulant_softmax_attention_amd/csrc/cat_fft.hpp",
                                "circulant_softmax_attention_amd/csrc/cat_common.hpp"]


def measured_traffic(kernel: str, workload: str, launches_per_call: int):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current sources of that kernel with the same launches per call;
    else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        if rec.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
            return None
        if rec.get("launches_per_call", 1) != launches_per_call:
            return None
        return rec.get("hbm_bytes_per_launch")
    except Exception:
        return None


def cpu_baseline(wl, inp, target_s: float, W_A=None):
    """The fp64 oracle, as it stands, on a bounded sample of the workload
    (W_A given: the CAT-scored 2D variant)."""
    import numpy as np

    import oracle
    threads = oracle.num_threads()
    if W_A is not None:
        # one head of one image end to end; a whole image is H such slices
        d = wl.d
        t0 = time.perf_counter()
        oracle.cat_scored_forward_2d(inp.X[:1], W_A[:, :1], inp.W_V[:, :d], wl.Hg, wl.Wg)
        secs = time.perf_counter() - t0
        return dict(cpu_model=cpu_model(), value=wl.N / (secs * wl.H), unit="tokens/s", cores=threads, kind="oracle",
                    sample=f"one head of one image (1/{wl.H} of an image, {wl.N} tokens) in {secs:.1f} s, "
                           f"scaled by {wl.H} heads per image; fp64 direct O(N^2 d) sums")
    if wl.kind == "1d" and wl.N > 4096:
        # one sequence's projections in full, and the circulant sum for a
        # sample of its rows; the time per token adds both shares
        t0 = time.perf_counter()
        oracle.scores_1d(inp.X[:1], inp.W_A)
        oracle.matmul(inp.X[:1], inp.W_V)
        t_proj = time.perf_counter() - t0
        zs = oracle.softmax(oracle.scores_1d(inp.X[:1], inp.W_A))
        V = oracle.matmul(inp.X[:1], inp.W_V)
        r = 64
        t0 = time.perf_counter()
        oracle.circulant_1d(zs, V, rows=list(range(r)))
        t_row = (time.perf_counter() - t0) / r
        per_token = t_proj / wl.N + t_row
        r = int(max(r, min(wl.N, (target_s - t_proj) / max(t_row, 1e-9))))
        t0 = time.perf_counter()
        oracle.circulant_1d(zs, V, rows=list(range(r)))
        t_row = (time.perf_counter() - t0) / r
        per_token = t_proj / wl.N + t_row
        return dict(cpu_model=cpu_model(), value=1.0 / per_token, unit="tokens/s", cores=threads, kind="oracle",
                    sample=f"projections of 1 sequence ({wl.N} tokens, {t_proj:.1f} s) and the fp64 direct "
                           f"circulant sum for {r} of its rows ({t_row * r:.1f} s); tokens/s = 1 / "
                           f"(projection time per token + sum time per row)")
    if wl.kind == "1d":
        t0 = time.perf_counter()
        oracle.cat_forward_1d(inp.X[:1], inp.W_A, inp.W_V)
        t1 = time.perf_counter() - t0
        n = int(max(1, min(wl.B - 1, round((target_s - t1) / max(t1, 1e-9)))))
        t0 = time.perf_counter()
        oracle.cat_forward_1d(inp.X[1:1 + n], inp.W_A, inp.W_V)
        tn = time.perf_counter() - t0
        imgs, secs = 1 + n, t1 + tn
        return dict(cpu_model=cpu_model(), value=imgs * wl.N / secs, unit="tokens/s", cores=threads, kind="oracle",
                    sample=f"{imgs} of {wl.B} sequences ({imgs * wl.N} tokens), fp64 direct O(N^2 d) sums, "
                           f"{secs:.1f} s")
    # 2D: one (image, head) slice end to end; a whole image is H such slices
    d = wl.d
    t0 = time.perf_counter()
    hs = slice(0, d)
    oracle.cat_forward_bccb_2d(inp.X[:1], inp.W_Q[:, hs], inp.W_K[:, hs], inp.W_V[:, hs], wl.Hg, wl.Wg, 1)
    secs = time.perf_counter() - t0
    per_image = secs * wl.H
    return dict(cpu_model=cpu_model(), value=wl.N / per_image, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"one head of one image (1/{wl.H} of an image, {wl.N} tokens) in {secs:.1f} s, "
                       f"scaled by {wl.H} heads per image; fp64 direct O(N^2 d) sums")


def timed_steps(step, K: int):
    """The timed region: K steps between synchronisations, with an event on
    the launch stream at every step boundary.  Returns the wall-clock mean
    (the headline's step time), the events' mean, and the per-step event
    durations (their median is reported beside the mean)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(K):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(K)]
    ms = wall * 1000.0 / K
    ev_ms = evs[0].elapsed_time(evs[K]) / K
    log(f"{K} steps: {ms * 1000:.1f} us/step wall, {ev_ms * 1000:.1f} us/step events, "
        f"median {sorted(per)[K // 2] * 1000:.1f} us")
    return ms, ev_ms, per


def step_stats(per):
    """Median and 10th / 90th percentiles of per-step event times (ms)."""
    q = sorted(per)
    n = len(q)
    return {"median": round(q[n // 2], 5), "p10": round(q[n // 10], 5), "p90": round(q[min(n - 1, (9 * n) // 10)], 5)}


def copy_bandwidth(nbytes: int = 1 << 30, reps: int = 10):
    """Measured device-to-device copy rate (GB/s, bytes read + written per
    second) of torch's copy kernel over two buffers far larger than the
    Infinity Cache: the attainable HBM rate on this machine, next to the 8 TB/s
    peak."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) / 1000.0 / reps
    del src, dst
    return round(2.0 * nbytes / secs / 1e9, 1)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def dtype_label(storage: str, conv_path: str) -> str:
    """What the path computes in: storage dtype, then the arithmetic of the
    projection and of the mixing; accumulation is fp32 everywhere."""
    if storage == "f32":
        return "f32 (fp32 MFMA GEMM, fp32 transforms)"
    mix = {"fft_matrix": "fp16-operand MFMA DFT products with per-line power-of-two scaling (1D), "
                         "bf16-operand MFMA DFT-matrix products (2D)",
           "direct": "bf16 MFMA direct product (softmax weights rounded to bf16)",
           "fft_valu": "fp32 vector-ALU transforms",
           "fft_multipass": "fp32 vector-ALU transforms, bf16-pair intermediates between the passes "
                            "where both sides are 64 or 256 points"}.get(conv_path, conv_path)
    return f"bf16 storage; bf16 MFMA GEMM; {mix}; fp32 accumulate"


def run(args):
    import numpy as np
    import torch

    from circulant_softmax_attention_amd import workloads as W
    lib_path = os.path.join(ROOT, "circulant_softmax_attention_amd", "libcat.so")
    if not os.path.exists(lib_path):
        from circulant_softmax_attention_amd import build
        build.build(verbose=False)
    from circulant_softmax_attention_amd import cat

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a ROCm GPU")
    wl = W.WORKLOADS[args.workload]
    log("workload", wl.name, wl.note)
    inp = W.make_inputs(wl)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).cuda()

    cat2d = args.variant == "cat2d"
    avgkey, causal = args.variant == "avgkey", args.variant == "causal"
    if cat2d and wl.kind != "2d":
        raise SystemExit("--variant cat2d runs on 2D workloads")
    if (avgkey or causal) and wl.kind != "1d":
        raise SystemExit(f"--variant {args.variant} runs on 1D workloads")
    if wl.kind == "1d":
        plan = cat.cat_plan_create("1d", wl.dtype, wl.B, wl.N, wl.D, wl.H)
        weights = [dev(inp.W_A), dev(inp.W_V)]
        if avgkey:
            # the averaged-key variant's W_Q and W_K by the workload's weight recipe (seeded)
            W_Q, W_K = W.extra_square_weights(wl, 2)
            weights = [dev(W_Q), dev(W_K), dev(inp.W_V)]
    else:
        plan = cat.cat_plan_create("2d", wl.dtype, wl.B, wl.N, wl.D, wl.H, wl.Hg, wl.Wg)
        weights = [dev(inp.W_Q), dev(inp.W_K), dev(inp.W_V)]
        if cat2d:
            # the CAT score projection by the workload's weight recipe (N(0, 1/D), seeded)
            W_A = np.random.default_rng(wl.seed + 1000).standard_normal((wl.D, wl.H)) / math.sqrt(wl.D)
            weights = [dev(W_A), dev(inp.W_V)]
    L, L1, L2 = plan.geometry()
    ws_bytes = plan.workspace_size()
    x0 = dev(inp.X)
    esz = 4 if wl.dtype == "f32" else 2
    set_bytes = 2 * x0.numel() * esz + ws_bytes
    nsets = max(1, math.ceil(args.rotate_bytes / set_bytes))
    X = [x0] + [x0.clone() for _ in range(nsets - 1)]
    O = [torch.empty_like(x0) for _ in range(nsets)]
    WS = [cat.alloc_workspace(plan) for _ in range(nsets)]
    log(f"transform {L} = {L1} x {L2}; {nsets} buffer sets of {set_bytes / 2**20:.1f} MiB")

    fwd = (cat.cat_forward_avgkey_1d if avgkey else cat.cat_forward_causal_1d if causal
           else cat.cat_forward_1d if wl.kind == "1d" else cat.cat_forward_cat_2d if cat2d else cat.cat_forward_bccb_2d)

    def step(i):
        k = i % nsets
        fwd(plan, X[k], *weights, O=O[k], workspace=WS[k])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    ms_per_step, gpu_ms_per_step, step_ms = timed_steps(step, args.steps)

    # instrumented pass, K more steps: the library launches every kernel with
    # start/stop events that its dispatch stamps (same stream as the kernel);
    # stamping serialises the kernels a little, so the step time of this pass
    # is reported separately and is not the headline number
    cat.cat_plan_set_timing(plan, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    inst_ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    ktimes = cat.cat_plan_kernel_times(plan)
    cat.cat_plan_set_timing(plan, False)
    conv_path = plan.conv_path()
    if causal:  # the causal direct product in the mixing slot
        ktimes["causalconv"] = ktimes.pop("fftconv")
    elif conv_path == "direct":  # the mixing launch is the direct product, not a transform
        ktimes["directconv"] = ktimes.pop("fftconv")
    if conv_path == "fft_matrix" and wl.Hg:  # 2D products on the matrix cores
        ktimes["fftconv_matrix"] = ktimes.pop("fftconv")
    for k, (ms, n) in ktimes.items():
        log(f"  kernel {k:10s} {ms * 1000:9.2f} us avg over {n} launches")

    ngrp = (wl.d // 2 + 1) // 2  # score partials per (batch, head): pairs in groups of 2
    fused = wl.kind == "1d" and ktimes.get("spectrum", (0.0, 0))[1] == 0
    # the CAT-scored 2D variant has the 1D launch structure (fused scores,
    # spectrum from logits, conv) on the 2D grid's transforms
    model = kernel_model(dataclasses.replace(wl, kind="1d") if cat2d else wl, L, ngrp,
                         fused_spectrum=fused and conv_path == "fft_matrix",
                         direct=conv_path == "direct", multipass=conv_path == "fft_multipass")
    T, s_ = wl.B * wl.N, (4 if wl.dtype == "f32" else 2)
    if avgkey:
        # V alone from the GEMM; the logits from four small launches (column
        # sums of X, the mean key, the per-head score weights, X . w):
        # X read twice, W_Q and W_K once, z written
        model["project"] = dict(bytes=2 * T * wl.D * s_ + wl.D * wl.D * s_, flops=2.0 * T * wl.D * wl.D,
                                unit=model["project"]["unit"])
        model["avgkey_logits"] = dict(bytes=2 * T * wl.D * s_ + 2 * wl.D * wl.D * s_ + wl.B * wl.H * wl.N * 4,
                                      flops=T * wl.D + 4.0 * wl.B * wl.D * wl.D + 2.0 * T * wl.D * wl.H, unit="valu_f32")
    if causal:
        # the masked direct product: N (N + 1) / 2 kept lags per (batch, head), 2 d flops each
        model["causalconv"] = dict(bytes=2 * T * wl.D * s_ + wl.B * wl.H * wl.N * 4,
                                   flops=1.0 * wl.B * wl.H * wl.N * (wl.N + 1) * wl.d,
                                   unit="mfma_bf16" if s_ == 2 else "mfma_f32")
    kernels = {}
    ktimes = {k: v for k, v in ktimes.items() if v[1] > 0}  # kernels this path launched
    for k, (ms, n) in ktimes.items():
        mm = model[k]
        per_call = max(1, round(n / args.steps))  # launches of this kernel per forward call
        sec = ms / 1000.0                          # average duration of one launch
        nbytes, nflops = mm["bytes"] / per_call, mm["flops"] / per_call
        gbs = nbytes / sec / 1e9
        tfl = nflops / sec / 1e12
        kernels[k] = dict(us=round(ms * 1000, 3), launches_per_call=per_call, bytes=int(nbytes), flops=float(nflops),
                          hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                          compute_frac=round(tfl / PEAK_TFLOPS[mm["unit"]], 4), compute_unit=mm["unit"])
    dom = max(ktimes, key=lambda k: ktimes[k][0] * kernels[k]["launches_per_call"])
    kd = kernels[dom]
    sec = ktimes[dom][0] / 1000.0
    if kd["compute_unit"].startswith("mfma") and kd["compute_frac"] >= kd["hbm_frac"]:
        bound = "mfma"
    else:
        bound = "hbm" if kd["hbm_frac"] >= kd["compute_frac"] else "alu"
    if bound == "hbm":
        achieved, peak, unit = kd["bytes"] / sec / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = kd["flops"] / sec / 1e12, PEAK_TFLOPS[kd["compute_unit"]], "TFLOP/s"
    roofline = dict(kernel=dom, bound=bound, achieved=round(achieved, 2), peak=peak, unit=unit,
                    frac=round(achieved / peak, 4), traffic=measured_traffic(dom, wl.name, kd["launches_per_call"]),
                    hbm_frac=kd["hbm_frac"], compute_frac=kd["compute_frac"], us=kd["us"])

    if wl.kind == "1d" and conv_path in ("fft_matrix", "direct") and args.variant is None:
        # the same mixing on the fp32 vector-ALU transforms (CAT_CONV=valu),
        # its kernels timed over K forward calls of a plan that takes them
        # (one buffer set; reported beside the step, not part of it)
        prev = os.environ.get("CAT_CONV")
        os.environ["CAT_CONV"] = "valu"
        try:
            vplan = cat.cat_plan_create("1d", wl.dtype, wl.B, wl.N, wl.D, wl.H)
        finally:
            if prev is None:
                os.environ.pop("CAT_CONV")
            else:
                os.environ["CAT_CONV"] = prev
        vws = cat.alloc_workspace(vplan)
        Ov = torch.empty_like(x0)
        for _ in range(3):
            cat.cat_forward_1d(vplan, X[0], *weights, O=Ov, workspace=vws)
        cat.cat_plan_set_timing(vplan, True)
        for _ in range(args.steps):
            cat.cat_forward_1d(vplan, X[0], *weights, O=Ov, workspace=vws)
        torch.cuda.synchronize()
        vt = cat.cat_plan_kernel_times(vplan)
        cat.cat_plan_set_timing(vplan, False)
        vmodel = kernel_model(wl, vplan.geometry()[0], ngrp)
        for k in ("spectrum", "fftconv"):
            ms, n = vt[k]
            if n:
                mm = vmodel[k]
                kernels[k + "_valu_f32"] = dict(us=round(ms * 1000, 3), launches_per_call=1, bytes=int(mm["bytes"]),
                                                flops=float(mm["flops"]),
                                                hbm_frac=round(mm["bytes"] / (ms / 1000) / 1e9 / HBM_PEAK_GBS, 4),
                                                compute_frac=round(mm["flops"] / (ms / 1000) / 1e12 / PEAK_TFLOPS["valu_f32"], 4),
                                                compute_unit="valu_f32", note="fp32 vector-ALU mixing (CAT_CONV=valu), "
                                                "not in the timed step")
                log(f"  kernel {k + '_valu_f32':18s} {ms * 1000:9.2f} us (fp32 vector path, not in the step)")
        del vplan

    copy_gbs = copy_bandwidth()
    log(f"device copy: {copy_gbs:.0f} GB/s")
    roofline["measured_copy_GBps"] = copy_gbs
    if roofline["unit"] == "GB/s":
        roofline["frac_of_copy"] = round(roofline["achieved"] / copy_gbs, 4)

    cpu = None
    if not args.no_cpu_baseline and not (avgkey or causal):
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(wl, inp, args.cpu_seconds, W_A=W_A if cat2d else None)
        log("cpu baseline:", cpu)

    tokens = wl.B * wl.N
    value = tokens / (ms_per_step / 1000.0)
    line = {
        "metric": "circulant-attention tokens/s at N=1024,D=768; % of HBM roofline (1 GPU)"
        if wl.name == W.HEADLINE and args.variant is None else f"CAT-scored 2D tokens/s ({wl.name})" if cat2d
        else f"averaged-key CAT tokens/s ({wl.name})" if avgkey else f"causal CAT tokens/s ({wl.name})" if causal
        else f"circulant-attention tokens/s ({wl.name})",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "step_ms_events": step_stats(step_ms),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_label(wl.dtype, conv_path),
        "data": "synthetic (seeded PCG64: X~N(0,1), W~N(0,1/D))",
        "config": {"workload": wl.name, "kind": "2d-cat-scored" if cat2d else f"1d-{args.variant}" if args.variant else wl.kind,
                   "B": wl.B, "N": wl.N, "D": wl.D, "H": wl.H,
                   "grid": [wl.Hg, wl.Wg] if wl.kind == "2d" else None, "storage": wl.dtype,
                   "transform": [L, L1, L2], "mixing": conv_path, "global_batch": wl.B, "seq_len": wl.N, "parallelism": "none"},
        "e2e_hbm_frac": round(((2 * tokens * wl.D * esz) + sum(w.numel() * esz for w in weights))
                              / (ms_per_step / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
        "gpu_event_ms_per_step": round(gpu_ms_per_step, 5),
        "instrumented_ms_per_step": round(inst_ms, 5),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    return line


def backward_model(wl, L: int, ngrp: int, fwd_model):
    """Algorithmic bytes and flops of each kernel of one mixing-backward call
    (all launches of a kind together).  dV runs as the forward mixing of the
    reversed logits, so its spectrum / conv entries are the forward's."""
    s = 4 if wl.dtype == "f32" else 2
    B, N, D, H, d = wl.B, wl.N, wl.D, wl.H, wl.d
    T, BH = B * N, B * H
    lines = BH * (d // 2)
    m = {k: v for k, v in fwd_model.items() if k in ("spectrum", "fftconv", "directconv")}
    m["reverse"] = dict(bytes=2 * BH * N * 4, flops=0.0, unit="valu_f32")
    # dO (for the dV mixing) and V (for the score gradient) to the blocked
    # layout in the storage dtype: read + write each
    m["relayout"] = dict(bytes=2 * (2 * T * D * s), flops=0.0, unit="valu_f32")
    # the blocked dO and V read once, the per-group partial spectra written
    m["score_grad"] = dict(bytes=2 * T * D * s + BH * ngrp * L * 8,
                           flops=lines * (2 * fft_flops(L) + 8.0 * L), unit="valu_f32")
    m["psum"] = dict(bytes=BH * ngrp * L * 8 + BH * L * 8, flops=2.0 * BH * (ngrp - 1) * L, unit="valu_f32")
    m["logits_grad"] = dict(bytes=BH * L * 8 + 2 * BH * N * 4, flops=BH * (fft_flops(L) + 8.0 * N), unit="valu_f32")
    return m


def run_backward(args):
    """The 1D mixing backward (dlogits, dV from logits, V and dO) on the
    workload's shapes: V and the logits from the projection of the workload's
    X, dO ~ N(0, 1) seeded."""
    import numpy as np
    import torch

    from circulant_softmax_attention_amd import workloads as W
    from circulant_softmax_attention_amd import cat

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a ROCm GPU")
    wl = W.WORKLOADS[args.workload]
    if wl.kind != "1d":
        raise SystemExit("--backward covers 1D workloads")
    log("workload", wl.name, "(mixing backward)")
    inp = W.make_inputs(wl)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).cuda()

    plan = cat.cat_plan_create("1d", wl.dtype, wl.B, wl.N, wl.D, wl.H)
    L, L1, L2 = plan.geometry()
    conv_path = plan.conv_path()
    V0, z0 = cat.cat_step_project(plan, dev(inp.X), dev(inp.W_A), dev(inp.W_V))
    g = np.random.default_rng(99).standard_normal((wl.B, wl.N, wl.D)).astype(np.float32)
    dO0 = dev(g)
    esz = 4 if wl.dtype == "f32" else 2
    ws_bytes = plan.workspace_size()
    set_bytes = 4 * V0.numel() * esz + 2 * z0.numel() * 4 + ws_bytes
    nsets = max(1, math.ceil(args.rotate_bytes / set_bytes))
    sets = []
    for i in range(nsets):
        sets.append((z0 if i == 0 else z0.clone(), V0 if i == 0 else V0.clone(), dO0 if i == 0 else dO0.clone(),
                     cat.alloc_workspace(plan)))
    log(f"transform {L} = {L1} x {L2}; mixing path {conv_path}; {nsets} buffer sets of {set_bytes / 2**20:.1f} MiB")

    full = args.backward == "full"
    Xd, WAd, WVd = dev(inp.X), dev(inp.W_A), dev(inp.W_V)

    def step(i):
        z, V, dO, ws = sets[i % nsets]
        if full:
            cat.cat_backward_1d(plan, Xd, WAd, WVd, dO, workspace=ws)
        else:
            cat.cat_step_mix_backward_1d(plan, z, V, dO, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step, gpu_ms_per_step, step_ms = timed_steps(step, args.steps)

    cat.cat_plan_set_timing(plan, True)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ktimes = {k: v for k, v in cat.cat_plan_kernel_times(plan).items() if v[1] > 0}
    cat.cat_plan_set_timing(plan, False)
    if full:
        ktimes.pop("project", None)  # the recompute GEMM; the gradient GEMMs are not in the timing slots
    if conv_path == "direct":
        ktimes["directconv"] = ktimes.pop("fftconv")
    ngrp = (wl.d // 2 + 1) // 2
    fwd = kernel_model(wl, L, ngrp, fused_spectrum=conv_path == "fft_matrix", direct=conv_path == "direct")
    model = backward_model(wl, L, ngrp, fwd)
    kernels = {}
    for k, (ms, n) in ktimes.items():
        mm = model[k]
        per_call = max(1, round(n / args.steps))
        sec = ms / 1000.0
        nbytes, nflops = mm["bytes"] / per_call, mm["flops"] / per_call
        kernels[k] = dict(us=round(ms * 1000, 3), launches_per_call=per_call, bytes=int(nbytes), flops=float(nflops),
                          hbm_frac=round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4),
                          compute_frac=round(nflops / sec / 1e12 / PEAK_TFLOPS[mm["unit"]], 4),
                          compute_unit=mm["unit"])
        log(f"  kernel {k:12s} {ms * 1000:9.2f} us avg over {n} launches ({per_call}/call)")
    dom = max(kernels, key=lambda k: kernels[k]["us"] * kernels[k]["launches_per_call"])
    kd = kernels[dom]
    sec = kd["us"] / 1e6
    if kd["compute_unit"].startswith("mfma") and kd["compute_frac"] >= kd["hbm_frac"]:
        bound, achieved, peak, unit = "mfma", kd["flops"] / sec / 1e12, PEAK_TFLOPS[kd["compute_unit"]], "TFLOP/s"
    elif kd["hbm_frac"] >= kd["compute_frac"]:
        bound, achieved, peak, unit = "hbm", kd["bytes"] / sec / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "alu", kd["flops"] / sec / 1e12, PEAK_TFLOPS[kd["compute_unit"]], "TFLOP/s"
    traffic = measured_traffic(dom, wl.name, kd["launches_per_call"]) if dom in KERNEL_SOURCES else None
    roofline = dict(kernel=dom, bound=bound, achieved=round(achieved, 2), peak=peak, unit=unit,
                    frac=round(achieved / peak, 4), traffic=traffic, hbm_frac=kd["hbm_frac"],
                    compute_frac=kd["compute_frac"], us=kd["us"])

    cpu = None
    if not args.no_cpu_baseline and not full:
        import oracle
        # whole sequences, one at a time, until about --cpu-seconds of work
        zc, Vc, gc = z0.cpu().numpy(), V0.float().cpu().numpy(), dO0.float().cpu().numpy()
        secs, nseq = 0.0, 0
        while nseq < wl.B and (nseq == 0 or secs < args.cpu_seconds):
            t0 = time.perf_counter()
            oracle.mix_backward_1d(zc[nseq:nseq + 1], Vc[nseq:nseq + 1], gc[nseq:nseq + 1])
            secs += time.perf_counter() - t0
            nseq += 1
        cpu = dict(cpu_model=cpu_model(), value=nseq * wl.N / secs, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                   sample=f"{nseq} of {wl.B} sequences ({nseq * wl.N} tokens), fp64 direct O(N^2 d) sums for dV "
                          f"and dz*, {secs:.1f} s")
        log("cpu baseline:", cpu)

    tokens = wl.B * wl.N
    io_bytes = 3 * tokens * wl.D * esz + 2 * wl.B * wl.H * wl.N * 4  # V, dO read, dV written; logits, dlogits
    return {
        "metric": f"CAT backward (dX, dW_A, dW_V) tokens/s ({wl.name})" if full
        else f"circulant mixing backward tokens/s ({wl.name})",
        "value": round(tokens / (ms_per_step / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "step_ms_events": step_stats(step_ms),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_label(wl.dtype, conv_path),
        "data": "synthetic (seeded PCG64: V, logits = projections of X~N(0,1); dO~N(0,1))",
        "gemm_flops_per_step": (2.0 * tokens * wl.D * (2 * wl.D + wl.H) + 2.0 * wl.D * tokens * (wl.D + (wl.H + 7) // 8 * 8))
        if full else None,
        "config": {"workload": wl.name, "kind": "1d-backward" if full else "1d-mix-backward", "B": wl.B, "N": wl.N, "D": wl.D, "H": wl.H,
                   "storage": wl.dtype, "transform": [L, L1, L2], "mixing": conv_path, "global_batch": wl.B,
                   "seq_len": wl.N, "parallelism": "none"},
        "e2e_hbm_frac": round(io_bytes / (ms_per_step / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
        "gpu_event_ms_per_step": round(gpu_ms_per_step, 5),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="workload name (default: the N=1024, D=768 one)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", choices=["cat2d", "avgkey", "causal"], default=None,
                    help="cat2d: the CAT-scored 2D variant (cat_forward_cat_2d) on a 2D workload; avgkey: the "
                         "averaged-key variant (cat_forward_avgkey_1d), causal: causal CAT (cat_forward_causal_1d), "
                         "on a 1D workload")
    ap.add_argument("--backward", nargs="?", const="mix", choices=["mix", "full"], default=None,
                    help="time a 1D backward instead of the forward: mix = cat_step_mix_backward_1d, "
                         "full = cat_backward_1d (dX, dW_A, dW_V)")
    ap.add_argument("--rotate-bytes", type=float, default=2.5 * MALL_BYTES,
                    help="total bytes of rotated buffer sets (defeats the Infinity Cache)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, --steps times (for scaling HBM counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(2)]
        dst = [torch.empty_like(src[0]) for _ in range(2)]
        for i in range(args.steps):
            dst[i % 2].copy_(src[i % 2])
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": args.steps}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path has no multi-GPU mode. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps > 256:
        print("--steps is limited to 256 (per-kernel timing slots)", file=sys.stderr)
        sys.exit(2)
    from circulant_softmax_attention_amd import workloads as W
    if args.workload is None:
        args.workload = W.HEADLINE
    line = run_backward(args) if args.backward else run(args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
