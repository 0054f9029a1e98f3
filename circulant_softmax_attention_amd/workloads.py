"""Workload table and seeded synthetic input generators.

This module holds no arithmetic of the method: it only names the problem
shapes and draws the random inputs (X and the projection weights) that both
the GPU path and the CPU oracle consume. Nothing here projects, normalises,
convolves or transforms.

Shapes follow the two pages' problem statements:
  * CAT: Circular-Convolutional Attention for Sub-Quadratic Transformers,
    "Method details / Overall framework": input X in R^{N x D}, a score
    projection W_A with one column per head ((D+H)·D parameters in total with
    W_V) and a value projection W_V in R^{D x D}.
  * Vision Transformers are Circulant Attention Learners, "Circulant
    Attention" section: Q, K, V projections of the patch tokens of an image,
    the tokens laid out on the patch grid.

Recipe (identical for every workload): a numpy Generator over PCG64 seeded
with the workload's seed draws, in fp64 and in this order, X ~ N(0, 1) with
shape [B, N, D]; then the score weights (W_A [D, H] for 1D, or W_Q then W_K,
each [D, D], for 2D) ~ N(0, 1/D); then W_V [D, D] ~ N(0, 1/D).  The draws are
cast to fp32 with numpy's round-to-nearest-even and, for bf16 storage, from
fp32 to bf16 with round-to-nearest-even.  The same rounded values go to the
oracle (upcast exactly) and to the GPU.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Workload:
    """One problem shape. For 2D, N = Hg * Wg tokens in raster order."""

    name: str
    kind: str  # "1d" or "2d"
    B: int
    N: int
    D: int
    H: int
    dtype: str  # storage dtype of X, weights and O: "f32" or "bf16"
    seed: int
    Hg: int = 0
    Wg: int = 0
    note: str = ""

    @property
    def d(self) -> int:
        return self.D // self.H

    @property
    def tokens(self) -> int:
        return self.B * self.N

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads, seeds 0..4 in this order.  The N=256 shape is run in two
# storage dtypes from the same draws.  Seed 5 is a long-sequence layer (the
# GPT-2-small shape at 65536 tokens), where the CAT page expects the
# O(N log N) route to pay; it measures the multi-pass path.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("cat1d_tiny_n64", "1d", 1, 64, 64, 4, F32, 0,
                 note="CAT 1D, B=1 N=64 D=64 H=4 (d=16), fp32"),
        Workload("cat1d_clipL_n256_f32", "1d", 64, 256, 1024, 16, F32, 1,
                 note="CAT 1D, CLIP-L/14 avg-pool layer shape (16x16 patches, no CLS), fp32"),
        Workload("cat1d_clipL_n256_bf16", "1d", 64, 256, 1024, 16, BF16, 1,
                 note="CAT 1D, CLIP-L/14 avg-pool layer shape, bf16 storage / fp32 compute"),
        Workload("cat1d_gpt2_n1024", "1d", 16, 1024, 768, 12, BF16, 2,
                 note="CAT 1D, GPT-2-small masked-LM layer shape, bf16 storage / fp32 compute"),
        Workload("cat1d_deitS_n197", "1d", 128, 197, 384, 6, F32, 3,
                 note="CAT 1D at prime length 197 (14x14 patches + CLS), DeiT-S shape, fp32"),
        Workload("bccb2d_1536px_96x96", "2d", 8, 96 * 96, 384, 6, BF16, 4, Hg=96, Wg=96,
                 note="2D BCCB circulant attention, 1536x1536 image at patch 16 (96x96 grid), bf16"),
        Workload("cat1d_long_n65536", "1d", 1, 65536, 768, 12, BF16, 5,
                 note="CAT 1D, GPT-2-small layer shape at N=65536 (multi-pass FFT), bf16 storage / fp32 compute"),
    ]
}

HEADLINE = "cat1d_gpt2_n1024"


def round_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) with round-to-nearest-even.

    NaN is not produced by the generators, so it is not special-cased.
    """
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exactly equal fp32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    """Storage-dtype inputs.  `*_bits` are uint16 bf16 patterns (bf16 only);
    the float32 arrays always hold the exact stored values."""

    wl: Workload
    X: np.ndarray
    W_V: np.ndarray
    W_A: Optional[np.ndarray] = None  # 1D
    W_Q: Optional[np.ndarray] = None  # 2D
    W_K: Optional[np.ndarray] = None  # 2D
    bits: Optional[Dict[str, np.ndarray]] = None

    def arrays(self) -> Dict[str, np.ndarray]:
        names = ["X", "W_A", "W_V"] if self.wl.kind == "1d" else ["X", "W_Q", "W_K", "W_V"]
        return {n: getattr(self, n) for n in names}


def _store(a64: np.ndarray, dtype: str):
    a32 = a64.astype(np.float32)
    if dtype == F32:
        return a32, None
    bits = round_bf16_bits(a32)
    return bf16_bits_to_f32(bits).reshape(a32.shape), bits.reshape(a32.shape)


def make_inputs(wl: Workload, seed: Optional[int] = None, batch: Optional[int] = None,
                x_scale: float = 1.0, score_scale: float = 1.0) -> Inputs:
    """Draw the inputs of `wl` with the recipe in the module docstring.

    `batch` overrides B.  X is drawn first, so with a different B the weights
    come from a different stream position than in the full workload; full-size
    parity therefore draws the full workload and slices it.  `score_scale` multiplies the score weights
    (W_A or W_Q, W_K) before rounding; 1.0 is the recipe, smaller values give
    a less peaked softmax for extra correctness cases.
    """
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    B = wl.B if batch is None else batch
    D, H = wl.D, wl.H
    std = 1.0 / np.sqrt(D)
    X = rng.standard_normal((B, wl.N, D)) * x_scale
    if wl.kind == "1d":
        WA = rng.standard_normal((D, H)) * std * score_scale
        WQ = WK = None
    else:
        WA = None
        WQ = rng.standard_normal((D, D)) * std * score_scale
        WK = rng.standard_normal((D, D)) * std * score_scale
    WV = rng.standard_normal((D, D)) * std
    out = {}
    bits = {}
    for name, a in [("X", X), ("W_A", WA), ("W_Q", WQ), ("W_K", WK), ("W_V", WV)]:
        if a is None:
            continue
        v, b = _store(a, wl.dtype)
        out[name] = v
        if b is not None:
            bits[name] = b
    return Inputs(wl=wl if batch is None else wl.with_(B=B), bits=bits or None, **out)


def extra_square_weights(wl: Workload, count: int, seed_offset: int = 1000):
    """`count` further [D, D] weights ~ N(0, 1/D) for the variants that need
    more projections than a workload's own (the averaged-key variant's W_Q
    and W_K on a 1D workload), from their own stream: PCG64 seeded with
    wl.seed + seed_offset, drawn in fp64 in order and stored like the
    workload's inputs."""
    rng = np.random.Generator(np.random.PCG64(wl.seed + seed_offset))
    std = 1.0 / np.sqrt(wl.D)
    return [_store(rng.standard_normal((wl.D, wl.D)) * std, wl.dtype)[0] for _ in range(count)]
