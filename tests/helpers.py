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


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(got, ref) -> float:
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))))


def assert_parity(got, ref, dtype: str, what: str = ""):
    r = rel_l2(got, ref)
    m = max_abs(got, ref)
    tol = TOL[dtype]
    msg = f"{what}: rel_l2={r:.3e} max_abs={m:.3e} (dtype {dtype})"
    assert r <= tol["rel"], msg
    if tol["abs"] is not None:
        assert m <= tol["abs"], msg
    return r, m


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
