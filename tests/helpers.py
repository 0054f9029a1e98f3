"""Shared test utilities: library availability, device tensors, parity metrics."""
from __future__ import annotations

import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "circulant_softmax_attention_amd", "libcat.so")

# Parity bars: fp32 storage -> rel L2 <= 1e-5 and max-abs <= 1e-4;
# bf16 storage (fp32 compute) -> rel L2 <= 2e-2.
TOL = {"f32": {"rel": 1e-5, "abs": 1e-4}, "bf16": {"rel": 2e-2, "abs": None}}


def ensure_lib():
    """Build libcat.so if it is not there (CPU container); never on import."""
    if not os.path.exists(LIB):
        from circulant_softmax_attention_amd import build
        build.build(verbose=False)
    return LIB


def _real(a, what: str) -> np.ndarray:
    a = np.asarray(a)
    if np.iscomplexobj(a):
        raise TypeError(f"{what} is complex: compare complex values through as_real_pairs()")
    return a.astype(np.float64)


def as_real_pairs(a) -> np.ndarray:
    """Complex array -> float64 array with a trailing (real, imag) axis, so
    that both parts enter the parity metrics."""
    a = np.asarray(a)
    return np.stack([a.real, a.imag], axis=-1).astype(np.float64)


def rel_l2(got, ref) -> float:
    got = _real(got, "got")
    ref = _real(ref, "ref")
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(got, ref) -> float:
    return float(np.max(np.abs(_real(got, "got") - _real(ref, "ref"))))


U32 = 2.0 ** -24  # unit roundoff of fp32


def sum_bar(K: int, rms_a: float, rms_b: float, eps_in: float = 1e-5, tail: float = 5.0) -> float:
    """Max-abs bar for entries of an fp32 product summed over K terms a_t b_t
    (the weight gradients, K = B N tokens).

    Accumulation: the running sum of K terms of random sign has size about
    sqrt(t) rms(a b) after t terms, and each of the (at most K) additions
    rounds it with a relative error up to u = 2^-24; independent roundings
    add in quadrature, sqrt(sum_t t) u rms(ab) = u K rms(ab) / sqrt(2).
    Inputs: b is itself a computed fp32 result held to relative L2 eps_in
    (the fp32 bar of the step that makes it), so its errors add
    sqrt(K) eps_in rms(a) rms(b).  rms(ab) <= rms(a) rms(b) for independent
    factors.  `tail` covers the largest of many entries (about 5 standard
    deviations).  Never tighter than the stated 1e-4 for unit-scale outputs.
    """
    per = (U32 * K / np.sqrt(2.0) + eps_in * np.sqrt(K)) * rms_a * rms_b
    return float(max(1e-4, tail * per))


def assert_parity(got, ref, dtype: str, what: str = ""):
    r = rel_l2(got, ref)
    m = max_abs(got, ref)
    tol = TOL[dtype]
    msg = f"{what}: rel_l2={r:.3e} max_abs={m:.3e} (dtype {dtype})"
    assert r <= tol["rel"], msg
    if tol["abs"] is not None:
        assert m <= tol["abs"], msg
    return r, m


def assert_spectrum_parity(got, ref, what: str = ""):
    """Complex spectra at the fp32 bar, real and imaginary parts both."""
    assert np.iscomplexobj(got) and np.iscomplexobj(ref), what
    return assert_parity(as_real_pairs(got), as_real_pairs(ref), "f32", what)


def to_dev(arr, dtype: str, device="cuda"):
    """numpy float32 array holding exactly representable storage values ->
    device tensor of the storage dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)  # exact: values are already bf16-representable
    return t.to(device)


def to_np(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy()
