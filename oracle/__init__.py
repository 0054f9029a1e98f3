"""fp64 CPU oracle for circulant softmax attention -- TEST INFRASTRUCTURE.

Only the test suite, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  The GPU library neither imports nor
links it, and this package imports nothing from the GPU library: the only
module both sides share is the seeded input generator, which holds none of
the method's arithmetic.

The heavy loops live in `cat_oracle.c` (plain direct sums in double
precision, no FFT); this module marshals numpy arrays into it and composes
the steps in the order the pages give:

  CAT (CAT: Circular-Convolutional Attention for Sub-Quadratic Transformers,
  "Method details / Overall framework" and "Key designs"):
      Z = X W_A  ->  Z* = softmax over the N tokens, per head
      V = X W_V  ->  O_h = circ(Z*_h) V_h,  C[i][j] = Z*[(i - j) mod N]

  Backward of the 1D mixing (CAT is trained end to end; the chain rule of
  the forward sums, written out as direct sums):
      dV_h = circ(Z*_h)^T G_h,   dZ*_h[k] = sum_c sum_i G[i][c] V[(i - k) mod N][c],
      dZ_h = Z*_h . (dZ*_h - <Z*_h, dZ*_h>)

  CAT-scored 2D variant: the CAT scores z = X W_A, softmaxed over the grid,
  as the filter of the 2D circular convolution below.

  Averaged-key variant (the ablation table's "qkv (Averaged-Key)" row):
      Q, K, V = X W_Q, X W_K, X W_V;  kbar_h = token mean of K_h
      z_h[n] = Q_h[n] . kbar_h / sqrt(d)  ->  softmax over n  ->  circ(.) V_h

  Causal CAT (the training-strategy note on causal language models): row i
  of circ(z_h) keeps the tokens j <= i and is softmaxed over them,
      O[i] = sum_{j<=i} exp(z[i - j]) V[j] / sum_{j<=i} exp(z[i - j])

  2D circulant attention (Vision Transformers are Circulant Attention
  Learners, "Circulant Attention: attention rebuilt with the FFT"):
      Q, K, V = X W_Q, X W_K, X W_V
      a_h = circular cross-correlation of Q_h and K_h on the token grid,
            summed over the head's channels, times 1/sqrt(d)
      O_h = BCCB(softmax(a_h)) V_h  (2D circular convolution)

Every function here is pinned by `tests/test_oracle.py` to something other
than itself (library routines on a different route, closed forms,
invariants, hand-computed fixtures in `tests/golden/`).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Dict, Optional, Sequence

import numpy as np

from . import build as _build

_lib = None
_P = ctypes.POINTER(ctypes.c_double)
_I64P = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is None:
        if _build.needs_build():
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_matmul.argtypes = [_P, _P, _P, _i64, _i64, _i64]
        lib.oracle_scores_1d.argtypes = [_P, _P, _P, _i64, _i64, _i64, _i64]
        lib.oracle_softmax_rows.argtypes = [_P, _P, _i64, _i64]
        lib.oracle_circulant_1d.argtypes = [_P, _P, _P, _i64, _i64, _i64, _i64, _I64P, _i64]
        lib.oracle_scores_bccb_2d.argtypes = [_P, _P, _P, _i64, _i64, _i64, _i64, _i64,
                                              ctypes.c_double]
        lib.oracle_bccb_2d.argtypes = [_P, _P, _P, _i64, _i64, _i64, _i64, _i64, _I64P, _i64]
        lib.oracle_circulant_1d_transpose.argtypes = [_P, _P, _P, _i64, _i64, _i64, _i64]
        lib.oracle_circulant_1d_grad_w.argtypes = [_P, _P, _P, _i64, _i64, _i64, _i64]
        lib.oracle_causal_1d.argtypes = [_P, _P, _P, _i64, _i64, _i64, _i64, _I64P, _i64]
        for f in ("oracle_matmul", "oracle_scores_1d", "oracle_softmax_rows",
                  "oracle_circulant_1d", "oracle_scores_bccb_2d", "oracle_bccb_2d",
                  "oracle_circulant_1d_transpose", "oracle_circulant_1d_grad_w", "oracle_causal_1d"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_P)


def _rows(rows: Optional[Sequence[int]]):
    if rows is None:
        return None, None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, r.ctypes.data_as(_I64P), int(r.size)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS or all cores)."""
    return int(_load().oracle_num_threads())


# ---------------------------------------------------------------- primitives
def matmul(X, W) -> np.ndarray:
    """[..., K] x [K, Nc] -> [..., Nc] in fp64 (X W, as the pages write it)."""
    X = _f64(X)
    W = _f64(W)
    K, Nc = W.shape
    assert X.shape[-1] == K
    M = X.size // K
    Y = np.empty(X.shape[:-1] + (Nc,), dtype=np.float64)
    _load().oracle_matmul(_ptr(X), _ptr(W), _ptr(Y), M, K, Nc)
    return Y


def scores_1d(X, W_A) -> np.ndarray:
    """z[b, h, n] = sum_k X[b, n, k] W_A[k, h]  ->  [B, H, N]."""
    X = _f64(X)
    W_A = _f64(W_A)
    B, N, D = X.shape
    H = W_A.shape[1]
    assert W_A.shape[0] == D
    z = np.empty((B, H, N), dtype=np.float64)
    _load().oracle_scores_1d(_ptr(X), _ptr(W_A), _ptr(z), B, N, D, H)
    return z


def softmax(z) -> np.ndarray:
    """Softmax over the last axis (max-subtracted)."""
    z = _f64(z)
    L = z.shape[-1]
    out = np.empty_like(z)
    _load().oracle_softmax_rows(_ptr(z), _ptr(out), z.size // max(L, 1), L)
    return out


def circulant_1d(w, V, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """O[b, i, c] = sum_j w[b, h(c), (i - j) mod N] V[b, j, c].

    w: [B, H, N]; V: [B, N, D].  Returns [B, N, D], or [len(rows), D] when
    `rows` (flattened b * N + i) is given.
    """
    w = _f64(w)
    V = _f64(V)
    B, H, N = w.shape
    assert V.shape[:2] == (B, N) and V.shape[2] % H == 0
    D = V.shape[2]
    r, rp, nr = _rows(rows)
    O = np.empty(((nr,) if r is not None else (B, N)) + (D,), dtype=np.float64)
    _load().oracle_circulant_1d(_ptr(w), _ptr(V), _ptr(O), B, N, D, H, rp, nr)
    return O


def scores_bccb_2d(Q, K, Hg: int, Wg: int, H: int, scale: Optional[float] = None) -> np.ndarray:
    """a[b, h, s1, s2]: circular cross-correlation of Q_h and K_h on the grid,
    summed over the head's d channels, times `scale` (default 1/sqrt(d))."""
    Q = _f64(Q)
    K = _f64(K)
    B, N, D = Q.shape
    assert K.shape == Q.shape and N == Hg * Wg and D % H == 0
    if scale is None:
        scale = 1.0 / math.sqrt(D // H)
    a = np.empty((B, H, Hg, Wg), dtype=np.float64)
    _load().oracle_scores_bccb_2d(_ptr(Q), _ptr(K), _ptr(a), B, Hg, Wg, D, H, float(scale))
    return a


def bccb_2d(w, V, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """O[b, (i1,i2), c] = sum_j w[b, h(c), (i1-j1) mod Hg, (i2-j2) mod Wg] V[b, j, c].

    w: [B, H, Hg, Wg]; V: [B, Hg*Wg, D]."""
    w = _f64(w)
    V = _f64(V)
    B, H, Hg, Wg = w.shape
    N = Hg * Wg
    assert V.shape[:2] == (B, N) and V.shape[2] % H == 0
    D = V.shape[2]
    r, rp, nr = _rows(rows)
    O = np.empty(((nr,) if r is not None else (B, N)) + (D,), dtype=np.float64)
    _load().oracle_bccb_2d(_ptr(w), _ptr(V), _ptr(O), B, Hg, Wg, D, H, rp, nr)
    return O


def circulant_1d_transpose(w, G) -> np.ndarray:
    """dV[b, j, c] = sum_i w[b, h(c), (i - j) mod N] G[b, i, c]: circ(w_h)^T G_h,
    the gradient of circulant_1d with respect to V for output gradient G."""
    w = _f64(w)
    G = _f64(G)
    B, H, N = w.shape
    assert G.shape[:2] == (B, N) and G.shape[2] % H == 0
    dV = np.empty_like(G)
    _load().oracle_circulant_1d_transpose(_ptr(w), _ptr(G), _ptr(dV), B, N, G.shape[2], H)
    return dV


def circulant_1d_grad_w(G, V, H: int) -> np.ndarray:
    """dw[b, h, k] = sum over the head's channels c and tokens i of
    G[b, i, c] V[b, (i - k) mod N, c]: the gradient of circulant_1d with
    respect to its filter w for output gradient G."""
    G = _f64(G)
    V = _f64(V)
    B, N, D = G.shape
    assert V.shape == G.shape and D % H == 0
    dw = np.empty((B, H, N), dtype=np.float64)
    _load().oracle_circulant_1d_grad_w(_ptr(G), _ptr(V), _ptr(dw), B, N, D, H)
    return dw


def causal_1d(z, V, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Causal CAT mixing from the logits z [B, H, N]:
    O[b, i, c] = sum_{j<=i} softmax_{j<=i}(z[b, h(c), i - j]) V[b, j, c],
    the row softmax of circ(z_h) with the tokens beyond i masked out.
    Returns [B, N, D], or [len(rows), D] for flattened rows b * N + i."""
    z = _f64(z)
    V = _f64(V)
    B, H, N = z.shape
    assert V.shape[:2] == (B, N) and V.shape[2] % H == 0
    D = V.shape[2]
    r, rp, nr = _rows(rows)
    O = np.empty(((nr,) if r is not None else (B, N)) + (D,), dtype=np.float64)
    _load().oracle_causal_1d(_ptr(z), _ptr(V), _ptr(O), B, N, D, H, rp, nr)
    return O


def avgkey_scores_1d(X, W_Q, W_K, H: int) -> np.ndarray:
    """Averaged-key logits [B, H, N]: with Q = X W_Q and K = X W_K, the key
    of head h is averaged over the N tokens, kbar_h = (1/N) sum_n K_h[n], and
    each token's query meets it as in scaled dot-product attention:
    z_h[n] = Q_h[n] . kbar_h / sqrt(d)  (d = D / H channels per head)."""
    X = _f64(X)
    B, N, D = X.shape
    d = D // H
    Q = matmul(X, W_Q).reshape(B, N, H, d)
    K = matmul(X, W_K).reshape(B, N, H, d)
    kbar = K.mean(axis=1)                                  # [B, H, d]
    z = (Q * kbar[:, None, :, :]).sum(axis=-1) / math.sqrt(d)  # [B, N, H]
    return np.ascontiguousarray(np.transpose(z, (0, 2, 1)))


def softmax_backward(zstar, g) -> np.ndarray:
    """dL/dz from g = dL/dz* through z* = softmax(z) over the last axis:
    z*_k (g_k - sum_m z*_m g_m)."""
    zstar = _f64(zstar)
    g = _f64(g)
    return zstar * (g - np.sum(zstar * g, axis=-1, keepdims=True))


# ---------------------------------------------------------------- composites
def mix_backward_1d(z, V, G) -> Dict[str, np.ndarray]:
    """Backward of the CAT mixing O_h = circ(softmax(z_h)) V_h for output
    gradient G: returns dz (logits gradient [B,H,N]) and dV ([B,N,D]).  The
    chain rule of the forward (CAT: Circular-Convolutional Attention for
    Sub-Quadratic Transformers, "Method details / Overall framework"):
    dV = circ(z*)^T G, dz* = circulant_1d_grad_w(G, V), dz = softmax'(dz*)."""
    z = _f64(z)
    zstar = softmax(z)
    dV = circulant_1d_transpose(zstar, G)
    dzs = circulant_1d_grad_w(G, V, z.shape[1])
    return {"dz": softmax_backward(zstar, dzs), "dV": dV, "dzstar": dzs}


def cat_backward_1d(X, W_A, W_V, G) -> Dict[str, np.ndarray]:
    """Gradients of the CAT forward (cat_forward_1d) for output gradient G:
    dX, dW_A, dW_V (and the mixing's dz, dV).  The chain rule through
    V = X W_V and z_h = X W_A[:, h]: dW_V = sum_b X_b^T dV_b,
    dW_A[k][h] = sum_{b,n} X[b][n][k] dz[b][h][n],
    dX = dV W_V^T + dz^T W_A^T."""
    X = _f64(X)
    W_A = _f64(W_A)
    W_V = _f64(W_V)
    z = scores_1d(X, W_A)
    V = matmul(X, W_V)
    mb = mix_backward_1d(z, V, G)
    dV, dz = mb["dV"], mb["dz"]
    B, N, D = X.shape
    Xf = X.reshape(B * N, D)
    dzt = np.transpose(dz, (0, 2, 1)).reshape(B * N, -1)  # [B*N, H]
    dW_V = matmul(Xf.T, dV.reshape(B * N, D))
    dW_A = matmul(Xf.T, dzt)
    dX = (matmul(dV.reshape(B * N, D), W_V.T) + matmul(dzt, W_A.T)).reshape(B, N, D)
    return {"dX": dX, "dW_A": dW_A, "dW_V": dW_V, "dz": dz, "dV": dV}


# ---------------------------------------------------------------- composites (forward)
def cat_forward_1d(X, W_A, W_V, rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """CAT forward: returns z (logits [B,H,N]), zstar (softmax), V (= X W_V) and O."""
    z = scores_1d(X, W_A)
    zstar = softmax(z)
    V = matmul(X, W_V)
    O = circulant_1d(zstar, V, rows=rows)
    return {"z": z, "zstar": zstar, "V": V, "O": O}


def cat_avgkey_forward_1d(X, W_Q, W_K, W_V, H: int, rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Averaged-key variant of CAT (CAT: Circular-Convolutional Attention for
    Sub-Quadratic Transformers, ablation table, row "qkv (Averaged-Key)":
    3 D^2 parameters, O(N log N)): the logits of avgkey_scores_1d, softmaxed
    over the N tokens, generate the circulant that mixes V = X W_V per head.
    Returns z, zstar, V and O."""
    z = avgkey_scores_1d(X, W_Q, W_K, H)
    zstar = softmax(z)
    V = matmul(X, W_V)
    O = circulant_1d(zstar, V, rows=rows)
    return {"z": z, "zstar": zstar, "V": V, "O": O}


def cat_causal_forward_1d(X, W_A, W_V, rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Causal CAT: the CAT logits z = X W_A, then causal_1d (each row of
    circ(z_h) masked to the tokens j <= i and softmaxed over them) applied
    to V = X W_V.  Returns z, V and O."""
    z = scores_1d(X, W_A)
    V = matmul(X, W_V)
    return {"z": z, "V": V, "O": causal_1d(z, V, rows=rows)}


def cat_scored_forward_2d(X, W_A, W_V, Hg: int, Wg: int, rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """CAT's scoring on a token grid: z = X W_A (one column per head),
    z* = softmax over all Hg*Wg tokens, O_h = BCCB(z*_h) V_h (2D circular
    convolution).  The circulant-attention page models the attention map as
    a BCCB matrix ("Circulant Attention: attention rebuilt with the FFT");
    here its filter comes from CAT's per-head score projection (CAT,
    "Method details / Overall framework") instead of the Q/K correlation.
    Returns z ([B,H,N]), zstar, V and O."""
    z = scores_1d(X, W_A)
    zstar = softmax(z)
    V = matmul(X, W_V)
    B, H, N = zstar.shape
    assert N == Hg * Wg
    O = bccb_2d(zstar.reshape(B, H, Hg, Wg), V, rows=rows)
    return {"z": z, "zstar": zstar, "V": V, "O": O}


def cat_forward_bccb_2d(X, W_Q, W_K, W_V, Hg: int, Wg: int, H: int,
                        rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """2D circulant attention forward: returns Q, K, V, a (scaled logits
    [B,H,Hg,Wg]), astar (softmax over all Hg*Wg positions) and O."""
    Q = matmul(X, W_Q)
    K = matmul(X, W_K)
    V = matmul(X, W_V)
    a = scores_bccb_2d(Q, K, Hg, Wg, H)
    B = a.shape[0]
    astar = softmax(a.reshape(B, H, Hg * Wg)).reshape(a.shape)
    O = bccb_2d(astar, V, rows=rows)
    return {"Q": Q, "K": K, "V": V, "a": a, "astar": astar, "O": O}
