"""Thin Python binding of libcat.so (include/cat.h).

Argument marshalling only: every function here checks the torch tensors it is
given (device, dtype, shape, contiguity), passes their device pointers and the
current HIP stream to the C entry point of the same name, and turns a non-OK
status into `CatError`.  All computation happens in the library's HIP
kernels.  There is no fallback: if libcat.so is missing or fails to load,
importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch  # loaded first so that libcat.so binds to the same HIP runtime

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcat.so")

CAT_OK = 0
STATUS_NAMES = {0: "CAT_OK", -1: "CAT_ERR_INVALID_ARG", -2: "CAT_ERR_UNSUPPORTED", -3: "CAT_ERR_HIP",
                -4: "CAT_ERR_ALLOC", -5: "CAT_ERR_PLAN_MISMATCH"}
CAT_F32, CAT_BF16 = 0, 1
CAT_1D, CAT_BCCB_2D = 0, 1

# Every symbol include/cat.h declares.
EXPORTS = ["cat_plan_create", "cat_plan_destroy", "cat_plan_workspace_size", "cat_plan_geometry",
           "cat_forward_1d", "cat_forward_bccb_2d", "cat_forward_cat_2d", "cat_status_string", "cat_last_error",
           "cat_plan_set_timing", "cat_plan_kernel_times", "cat_plan_conv_path",
           "cat_step_project", "cat_step_spectrum", "cat_step_mix", "cat_step_mix_backward_1d",
           "cat_backward_1d", "cat_step_scores_2d", "cat_forward_avgkey_1d", "cat_step_avgkey_logits",
           "cat_forward_causal_1d", "cat_step_mix_causal_1d", "cat_forward_1d_noalloc"]
KERNELS_1D = ["project", "spectrum", "fftconv", "reverse", "relayout", "score_grad", "psum", "logits_grad",
              "avgkey_logits"]
KERNELS_2D = ["project", "scores", "spectrum", "fftconv", "psum"]


class CatError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {message}")


class _Problem(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("dtype", ctypes.c_int32), ("B", ctypes.c_int64),
                ("N", ctypes.c_int64), ("D", ctypes.c_int64), ("H", ctypes.c_int64),
                ("Hg", ctypes.c_int64), ("Wg", ctypes.c_int64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m circulant_softmax_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    lib.cat_plan_create.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(_Problem)]
    lib.cat_plan_destroy.argtypes = [vp]
    lib.cat_plan_workspace_size.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    lib.cat_plan_geometry.argtypes = [vp] + [ctypes.POINTER(ctypes.c_int64)] * 3
    lib.cat_forward_1d.argtypes = [vp] * 7
    lib.cat_forward_bccb_2d.argtypes = [vp] * 8
    lib.cat_forward_cat_2d.argtypes = [vp] * 7
    lib.cat_plan_set_timing.argtypes = [vp, ctypes.c_int]
    lib.cat_plan_conv_path.argtypes = [vp, ctypes.POINTER(ctypes.c_int)]
    lib.cat_plan_kernel_times.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_int)]
    lib.cat_step_project.argtypes = [vp] * 9
    lib.cat_step_spectrum.argtypes = [vp] * 5
    lib.cat_step_mix.argtypes = [vp] * 6
    lib.cat_step_mix_backward_1d.argtypes = [vp] * 8
    lib.cat_backward_1d.argtypes = [vp] * 10
    lib.cat_step_scores_2d.argtypes = [vp] * 6
    lib.cat_forward_avgkey_1d.argtypes = [vp] * 8
    lib.cat_step_avgkey_logits.argtypes = [vp] * 7
    lib.cat_forward_causal_1d.argtypes = [vp] * 7
    lib.cat_step_mix_causal_1d.argtypes = [vp] * 6
    lib.cat_forward_1d_noalloc.argtypes = [vp] * 6
    for f in EXPORTS:
        fn = getattr(lib, f)
        if f in ("cat_status_string", "cat_last_error"):
            fn.restype = ctypes.c_char_p
        else:
            fn.restype = ctypes.c_int
    lib.cat_status_string.argtypes = [ctypes.c_int]
    lib.cat_last_error.argtypes = []
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _check(status: int, where: str):
    if status != CAT_OK:
        raise CatError(status, where, _lib.cat_last_error().decode())


def _dtype_code(dtype) -> int:
    if dtype in (torch.float32, "f32", "float32"):
        return CAT_F32
    if dtype in (torch.bfloat16, "bf16", "bfloat16"):
        return CAT_BF16
    raise ValueError(f"unsupported storage dtype {dtype}")


@dataclass
class Plan:
    """Owns a cat_plan handle."""

    handle: int
    kind: int
    dtype: torch.dtype
    B: int
    N: int
    D: int
    H: int
    Hg: int = 0
    Wg: int = 0

    def workspace_size(self) -> int:
        return cat_plan_workspace_size(self)

    def geometry(self):
        return cat_plan_geometry(self)

    def conv_path(self) -> str:
        return cat_plan_conv_path(self)

    def __del__(self):
        if getattr(self, "handle", None):
            _lib.cat_plan_destroy(ctypes.c_void_p(self.handle))
            self.handle = 0


def cat_plan_create(kind: str, dtype, B: int, N: int, D: int, H: int, Hg: int = 0, Wg: int = 0) -> Plan:
    code = _dtype_code(dtype)
    k = {"1d": CAT_1D, "2d": CAT_BCCB_2D}[kind]
    prob = _Problem(k, code, B, N, D, H, Hg, Wg)
    h = ctypes.c_void_p()
    _check(_lib.cat_plan_create(ctypes.byref(h), ctypes.byref(prob)), "cat_plan_create")
    return Plan(h.value, k, torch.float32 if code == CAT_F32 else torch.bfloat16, B, N, D, H, Hg, Wg)


def cat_plan_workspace_size(plan: Plan) -> int:
    n = ctypes.c_size_t()
    _check(_lib.cat_plan_workspace_size(ctypes.c_void_p(plan.handle), ctypes.byref(n)), "cat_plan_workspace_size")
    return int(n.value)


def cat_plan_geometry(plan: Plan):
    L, L1, L2 = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.cat_plan_geometry(ctypes.c_void_p(plan.handle), ctypes.byref(L), ctypes.byref(L1),
                                  ctypes.byref(L2)), "cat_plan_geometry")
    return int(L.value), int(L1.value), int(L2.value)


CONV_PATHS = {0: "fft_valu", 1: "fft_matrix", 2: "direct", 3: "fft_multipass"}


def cat_plan_conv_path(plan: Plan) -> str:
    """How the plan evaluates the circulant mixing: "fft_valu", "fft_matrix",
    "direct" or "fft_multipass" (include/cat.h, cat_plan_conv_path)."""
    p = ctypes.c_int()
    _check(_lib.cat_plan_conv_path(ctypes.c_void_p(plan.handle), ctypes.byref(p)), "cat_plan_conv_path")
    return CONV_PATHS[int(p.value)]


def cat_plan_set_timing(plan: Plan, enable: bool = True):
    _check(_lib.cat_plan_set_timing(ctypes.c_void_p(plan.handle), int(bool(enable))), "cat_plan_set_timing")


def cat_plan_kernel_times(plan: Plan):
    """{kernel name: (average ms per launch, launches)} over the calls recorded
    since timing was enabled."""
    tot = (ctypes.c_double * 16)()
    cnt = (ctypes.c_int64 * 16)()
    nk = ctypes.c_int()
    _check(_lib.cat_plan_kernel_times(ctypes.c_void_p(plan.handle), tot, cnt, ctypes.byref(nk)),
           "cat_plan_kernel_times")
    names = KERNELS_1D if plan.kind == CAT_1D else KERNELS_2D
    return {names[k]: ((tot[k] / cnt[k]) if cnt[k] else float("nan"), int(cnt[k])) for k in range(nk.value)}


def alloc_workspace(plan: Plan, device="cuda") -> torch.Tensor:
    return torch.empty(max(plan.workspace_size(), 256), dtype=torch.uint8, device=device)


def _stream_ptr(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor], shape=None, dtype=None, name="tensor") -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(None)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def cat_forward_1d(plan: Plan, X, W_A, W_V, O=None, workspace=None, stream=None) -> torch.Tensor:
    """O = CAT(X) per include/cat.h (W_A [D, H], W_V [D, D]); allocates
    O/workspace only when not given."""
    B, N, D, H, dt = plan.B, plan.N, plan.D, plan.H, plan.dtype
    if O is None:
        O = torch.empty((B, N, D), dtype=dt, device=X.device)
    if workspace is None:
        workspace = alloc_workspace(plan, X.device)
    _check(_lib.cat_forward_1d(ctypes.c_void_p(plan.handle), _ptr(X, (B, N, D), dt, "X"),
                               _ptr(W_A, (D, H), dt, "W_A"), _ptr(W_V, (D, D), dt, "W_V"),
                               _ptr(O, (B, N, D), dt, "O"), _ptr(workspace, None, None, "workspace"),
                               _stream_ptr(stream)), "cat_forward_1d")
    return O


def cat_forward_1d_noalloc(plan: Plan, X, W_A, W_V, O=None, stream=None) -> torch.Tensor:
    """cat_forward_1d on the library's fixed device scratch (no workspace);
    allocates O only when not given."""
    B, N, D, H, dt = plan.B, plan.N, plan.D, plan.H, plan.dtype
    if O is None:
        O = torch.empty((B, N, D), dtype=dt, device=X.device)
    _check(_lib.cat_forward_1d_noalloc(ctypes.c_void_p(plan.handle), _ptr(X, (B, N, D), dt, "X"),
                                       _ptr(W_A, (D, H), dt, "W_A"), _ptr(W_V, (D, D), dt, "W_V"),
                                       _ptr(O, (B, N, D), dt, "O"), _stream_ptr(stream)), "cat_forward_1d_noalloc")
    return O


def cat_forward_bccb_2d(plan: Plan, X, W_Q, W_K, W_V, O=None, workspace=None, stream=None) -> torch.Tensor:
    """O = 2D BCCB circulant attention(X) per include/cat.h (weights [D, D])."""
    B, N, D, dt = plan.B, plan.N, plan.D, plan.dtype
    if O is None:
        O = torch.empty((B, N, D), dtype=dt, device=X.device)
    if workspace is None:
        workspace = alloc_workspace(plan, X.device)
    _check(_lib.cat_forward_bccb_2d(ctypes.c_void_p(plan.handle), _ptr(X, (B, N, D), dt, "X"),
                                    _ptr(W_Q, (D, D), dt, "W_Q"), _ptr(W_K, (D, D), dt, "W_K"),
                                    _ptr(W_V, (D, D), dt, "W_V"), _ptr(O, (B, N, D), dt, "O"),
                                    _ptr(workspace, None, None, "workspace"), _stream_ptr(stream)),
           "cat_forward_bccb_2d")
    return O


def cat_forward_cat_2d(plan: Plan, X, W_A, W_V, O=None, workspace=None, stream=None) -> torch.Tensor:
    """O = the CAT-scored 2D variant per include/cat.h (W_A [D, H], W_V [D, D])."""
    B, N, D, H, dt = plan.B, plan.N, plan.D, plan.H, plan.dtype
    if O is None:
        O = torch.empty((B, N, D), dtype=dt, device=X.device)
    if workspace is None:
        workspace = alloc_workspace(plan, X.device)
    _check(_lib.cat_forward_cat_2d(ctypes.c_void_p(plan.handle), _ptr(X, (B, N, D), dt, "X"),
                                   _ptr(W_A, (D, H), dt, "W_A"), _ptr(W_V, (D, D), dt, "W_V"),
                                   _ptr(O, (B, N, D), dt, "O"), _ptr(workspace, None, None, "workspace"),
                                   _stream_ptr(stream)), "cat_forward_cat_2d")
    return O


def cat_step_project(plan: Plan, X, W_A, W_V, W_K=None, stream=None):
    """1D: returns (V [B,N,D] storage dtype, z [B,H,N] fp32).
    2D (W_A is W_Q): returns (Q fp32, K fp32, V storage dtype), all [B,N,D]."""
    B, N, D, H, dt = plan.B, plan.N, plan.D, plan.H, plan.dtype
    dev = X.device
    V = torch.empty((B, N, D), dtype=dt, device=dev)
    if plan.kind == CAT_1D:
        z = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        _check(_lib.cat_step_project(ctypes.c_void_p(plan.handle), _ptr(X, (B, N, D), dt, "X"),
                                     _ptr(W_A, (D, H), dt, "W_A"), ctypes.c_void_p(None),
                                     _ptr(W_V, (D, D), dt, "W_V"), _ptr(V), _ptr(z), ctypes.c_void_p(None),
                                     _stream_ptr(stream)), "cat_step_project")
        return V, z
    Q = torch.empty((B, N, D), dtype=torch.float32, device=dev)
    K = torch.empty((B, N, D), dtype=torch.float32, device=dev)
    _check(_lib.cat_step_project(ctypes.c_void_p(plan.handle), _ptr(X, (B, N, D), dt, "X"),
                                 _ptr(W_A, (D, D), dt, "W_Q"), _ptr(W_K, (D, D), dt, "W_K"),
                                 _ptr(W_V, (D, D), dt, "W_V"), _ptr(V), _ptr(Q), _ptr(K),
                                 _stream_ptr(stream)), "cat_step_project")
    return Q, K, V


def cat_step_spectrum(plan: Plan, logits, want_probs: bool = True, stream=None):
    """Returns (probs [B,H,N] fp32 or None, spec [B,H,L] complex64)."""
    B, N, H = plan.B, plan.N, plan.H
    L, _, _ = plan.geometry()
    probs = torch.empty((B, H, N), dtype=torch.float32, device=logits.device) if want_probs else None
    spec = torch.empty((B, H, L, 2), dtype=torch.float32, device=logits.device)
    _check(_lib.cat_step_spectrum(ctypes.c_void_p(plan.handle), _ptr(logits, (B, H, N), torch.float32, "logits"),
                                  _ptr(probs), _ptr(spec), _stream_ptr(stream)), "cat_step_spectrum")
    return probs, torch.view_as_complex(spec)


def cat_step_mix(plan: Plan, logits, V, O=None, workspace=None, stream=None) -> torch.Tensor:
    B, N, D, H, dt = plan.B, plan.N, plan.D, plan.H, plan.dtype
    if O is None:
        O = torch.empty((B, N, D), dtype=dt, device=V.device)
    if workspace is None:
        workspace = alloc_workspace(plan, V.device)
    _check(_lib.cat_step_mix(ctypes.c_void_p(plan.handle), _ptr(logits, (B, H, N), torch.float32, "logits"),
                             _ptr(V, (B, N, D), dt, "V"), _ptr(O, (B, N, D), dt, "O"), _ptr(workspace),
                             _stream_ptr(stream)), "cat_step_mix")
    return O


def cat_step_mix_backward_1d(plan: Plan, logits, V, dO, workspace=None, stream=None):
    """(dlogits [B,H,N] fp32, dV [B,N,D] storage dtype) for output gradient dO."""
    B, N, D, H, dt = plan.B, plan.N, plan.D, plan.H, plan.dtype
    if workspace is None:
        workspace = alloc_workspace(plan, V.device)
    dlogits = torch.empty((B, H, N), dtype=torch.float32, device=V.device)
    dV = torch.empty((B, N, D), dtype=dt, device=V.device)
    _check(_lib.cat_step_mix_backward_1d(ctypes.c_void_p(plan.handle),
                                         _ptr(logits, (B, H, N), torch.float32, "logits"),
                                         _ptr(V, (B, N, D), dt, "V"), _ptr(dO, (B, N, D), dt, "dO"),
                                         _ptr(dlogits), _ptr(dV), _ptr(workspace), _stream_ptr(stream)),
           "cat_step_mix_backward_1d")
    return dlogits, dV


def cat_backward_1d(plan: Plan, X, W_A, W_V, dO, workspace=None, stream=None):
    """(dX [B,N,D], dW_A [D,H], dW_V [D,D]), storage dtype, for output gradient dO."""
    B, N, D, H, dt = plan.B, plan.N, plan.D, plan.H, plan.dtype
    if workspace is None:
        workspace = alloc_workspace(plan, X.device)
    dX = torch.empty((B, N, D), dtype=dt, device=X.device)
    dW_A = torch.empty((D, H), dtype=dt, device=X.device)
    dW_V = torch.empty((D, D), dtype=dt, device=X.device)
    _check(_lib.cat_backward_1d(ctypes.c_void_p(plan.handle), _ptr(X, (B, N, D), dt, "X"), _ptr(W_A, (D, H), dt, "W_A"),
                                _ptr(W_V, (D, D), dt, "W_V"), _ptr(dO, (B, N, D), dt, "dO"), _ptr(dX), _ptr(dW_A),
                                _ptr(dW_V), _ptr(workspace), _stream_ptr(stream)), "cat_backward_1d")
    return dX, dW_A, dW_V


def cat_forward_avgkey_1d(plan: Plan, X, W_Q, W_K, W_V, O=None, workspace=None, stream=None) -> torch.Tensor:
    """O = the averaged-key variant of CAT per include/cat.h (weights [D, D])."""
    B, N, D, dt = plan.B, plan.N, plan.D, plan.dtype
    if O is None:
        O = torch.empty((B, N, D), dtype=dt, device=X.device)
    if workspace is None:
        workspace = alloc_workspace(plan, X.device)
    _check(_lib.cat_forward_avgkey_1d(ctypes.c_void_p(plan.handle), _ptr(X, (B, N, D), dt, "X"),
                                      _ptr(W_Q, (D, D), dt, "W_Q"), _ptr(W_K, (D, D), dt, "W_K"),
                                      _ptr(W_V, (D, D), dt, "W_V"), _ptr(O, (B, N, D), dt, "O"),
                                      _ptr(workspace, None, None, "workspace"), _stream_ptr(stream)),
           "cat_forward_avgkey_1d")
    return O


def cat_step_avgkey_logits(plan: Plan, X, W_Q, W_K, workspace=None, stream=None) -> torch.Tensor:
    """z [B, H, N] fp32: the averaged-key logits."""
    B, N, D, H, dt = plan.B, plan.N, plan.D, plan.H, plan.dtype
    if workspace is None:
        workspace = alloc_workspace(plan, X.device)
    z = torch.empty((B, H, N), dtype=torch.float32, device=X.device)
    _check(_lib.cat_step_avgkey_logits(ctypes.c_void_p(plan.handle), _ptr(X, (B, N, D), dt, "X"),
                                       _ptr(W_Q, (D, D), dt, "W_Q"), _ptr(W_K, (D, D), dt, "W_K"), _ptr(z),
                                       _ptr(workspace, None, None, "workspace"), _stream_ptr(stream)),
           "cat_step_avgkey_logits")
    return z


def cat_forward_causal_1d(plan: Plan, X, W_A, W_V, O=None, workspace=None, stream=None) -> torch.Tensor:
    """O = causal CAT per include/cat.h (W_A [D, H], W_V [D, D])."""
    B, N, D, H, dt = plan.B, plan.N, plan.D, plan.H, plan.dtype
    if O is None:
        O = torch.empty((B, N, D), dtype=dt, device=X.device)
    if workspace is None:
        workspace = alloc_workspace(plan, X.device)
    _check(_lib.cat_forward_causal_1d(ctypes.c_void_p(plan.handle), _ptr(X, (B, N, D), dt, "X"),
                                      _ptr(W_A, (D, H), dt, "W_A"), _ptr(W_V, (D, D), dt, "W_V"),
                                      _ptr(O, (B, N, D), dt, "O"), _ptr(workspace, None, None, "workspace"),
                                      _stream_ptr(stream)), "cat_forward_causal_1d")
    return O


def cat_step_mix_causal_1d(plan: Plan, logits, V, O=None, workspace=None, stream=None) -> torch.Tensor:
    B, N, D, H, dt = plan.B, plan.N, plan.D, plan.H, plan.dtype
    if O is None:
        O = torch.empty((B, N, D), dtype=dt, device=V.device)
    if workspace is None:
        workspace = alloc_workspace(plan, V.device)
    _check(_lib.cat_step_mix_causal_1d(ctypes.c_void_p(plan.handle),
                                       _ptr(logits, (B, H, N), torch.float32, "logits"), _ptr(V, (B, N, D), dt, "V"),
                                       _ptr(O, (B, N, D), dt, "O"), _ptr(workspace), _stream_ptr(stream)),
           "cat_step_mix_causal_1d")
    return O


def cat_step_scores_2d(plan: Plan, Q, K, workspace=None, stream=None) -> torch.Tensor:
    B, N, D, H = plan.B, plan.N, plan.D, plan.H
    if workspace is None:
        workspace = alloc_workspace(plan, Q.device)
    probs = torch.empty((B, H, N), dtype=torch.float32, device=Q.device)
    _check(_lib.cat_step_scores_2d(ctypes.c_void_p(plan.handle), _ptr(Q, (B, N, D), torch.float32, "Q"),
                                   _ptr(K, (B, N, D), torch.float32, "K"), _ptr(probs), _ptr(workspace),
                                   _stream_ptr(stream)), "cat_step_scores_2d")
    return probs
