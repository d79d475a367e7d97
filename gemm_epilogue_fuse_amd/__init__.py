"""libfuse: fused GEMM + epilogue and RMSNorm -> Linear on AMD MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/fuse.h``.  It only checks
and marshals arguments (dtype, device, contiguity, shapes) and passes raw
device pointers plus the current HIP stream; every step of the computation
runs in the HIP kernels of ``libfuse.so``.  PyTorch supplies device memory and
streams.  There is no fallback: if ``libfuse.so`` is missing or cannot be
loaded, every call raises.

Build the library with ``python -m gemm_epilogue_fuse_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "gemm_epilogue", "rmsnorm_gemm", "rmsnorm_gemm_swiglu", "swiglu_ffn", "plan_name", "set_plan",
    "workspace_bytes", "layernorm_gemm", "gemm_prologue_bias",
    "FuseError", "lib", "LIB_PATH", "ACT", "F16", "BF16", "OUT_F32",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfuse.so")

ACT = {"none": 0, "relu": 1, "gelu_tanh": 2, "silu": 3}
F16, BF16, OUT_F32 = 0, 1, 0x100
OP_GEMM, OP_RMS_GEMM, OP_RMS_SWIGLU, OP_LN_GEMM, OP_BIAS_GEMM = 0, 1, 2, 3, 4

_lib = None


class FuseError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = lib().fuse_strerror(status).decode()
        if status == 7:
            msg += ", hipError_t %d" % lib().fuse_last_hip_error()
        super().__init__("%s failed: status %d (%s)" % (what, status, msg))
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libfuse.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfuse.so not found at %s; build it with "
                               "`python -m gemm_epilogue_fuse_amd.build`" % LIB_PATH)
        # libfuse must run on the same HIP runtime instance that owns the
        # caller's memory and streams.  torch's HIP libraries ask for the
        # runtime by file name while libfuse asks by soname, so torch is loaded
        # first: libfuse then binds to the runtime already in the process
        # instead of pulling in a second one.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.fuse_gemm_epilogue.restype = ci
        L.fuse_gemm_epilogue.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ci, ci, vp]
        L.fuse_rmsnorm_gemm.restype = ci
        L.fuse_rmsnorm_gemm.argtypes = [vp, vp, ctypes.c_float, vp, vp, vp, i64, i64, i64, ci, ci, vp]
        L.fuse_rmsnorm_gemm_noalloc.restype = ci
        L.fuse_rmsnorm_gemm_noalloc.argtypes = [vp, vp, ctypes.c_float, vp, vp, vp, i64, i64, i64, ci, ci, vp]
        L.fuse_layernorm_gemm.restype = ci
        L.fuse_layernorm_gemm.argtypes = [vp, vp, vp, ctypes.c_float, vp, vp, vp, i64, i64, i64, ci, ci, vp]
        L.fuse_gemm_prologue_bias.restype = ci
        L.fuse_gemm_prologue_bias.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, ci, ci, vp]
        L.fuse_rmsnorm_gemm_swiglu.restype = ci
        L.fuse_rmsnorm_gemm_swiglu.argtypes = [vp, vp, ctypes.c_float, vp, vp, vp, i64, i64, i64, ci, vp]
        L.fuse_plan_name.restype = ctypes.c_char_p
        L.fuse_plan_name.argtypes = [ci, i64, i64, i64, ci]
        L.fuse_workspace_bytes.restype = i64
        L.fuse_workspace_bytes.argtypes = [ci, i64, i64, i64, ci]
        L.fuse_set_plan.restype = ci
        L.fuse_set_plan.argtypes = [ctypes.c_char_p]
        L.fuse_tune_set.restype = ci
        L.fuse_tune_set.argtypes = [ci, i64, i64, i64, ci, ctypes.c_char_p]
        L.fuse_tune_clear.restype = ci
        L.fuse_tune_clear.argtypes = []
        L.fuse_plan_count.restype = ci
        L.fuse_plan_count.argtypes = []
        L.fuse_plan_info.restype = ctypes.c_char_p
        L.fuse_plan_info.argtypes = [ci, ctypes.POINTER(ctypes.c_int32)]
        L.fuse_plan_applies.restype = ci
        L.fuse_plan_applies.argtypes = [ci, i64, i64, i64, ci, ctypes.c_char_p]
        L.fuse_kernel_resources.restype = ci
        L.fuse_kernel_resources.argtypes = [ci, i64, i64, i64, ci, ctypes.POINTER(ctypes.c_int32)]
        L.fuse_strerror.restype = ctypes.c_char_p
        L.fuse_strerror.argtypes = [ci]
        L.fuse_version.restype = ci
        L.fuse_version.argtypes = []
        L.fuse_last_hip_error.restype = ci
        L.fuse_last_hip_error.argtypes = []
        _lib = L
        # tuned plans from a persistent cache, when the environment names one
        cache = os.environ.get("LIBFUSE_TUNE_CACHE")
        if cache and os.path.exists(cache):
            from . import tuner
            tuner.load_cache(cache)
    return _lib


def _torch():
    import torch
    return torch


def _dtype_code(t, out_dtype) -> int:
    torch = _torch()
    if t.device.type != "cuda":
        raise ValueError("libfuse runs on the GPU only; got a tensor on %s" % t.device)
    if not t.is_contiguous():
        raise ValueError("inputs must be contiguous")
    if t.dtype == torch.float16:
        code = F16
    elif t.dtype == torch.bfloat16:
        code = BF16
    else:
        raise TypeError("inputs must be float16 or bfloat16, got %s" % t.dtype)
    if out_dtype is None or out_dtype == t.dtype:
        return code
    if out_dtype == torch.float32:
        return code | OUT_F32
    raise TypeError("output dtype must be the input dtype or float32")


def _check(t, name, dtype, shape, device):
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t


def _stream(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def _out(out, shape, dtype, device, name="out"):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _check(out, name, dtype, shape, device)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _act(act) -> int:
    if isinstance(act, str):
        if act not in ACT:
            raise ValueError("unknown activation %r" % act)
        return ACT[act]
    return int(act)


def gemm_epilogue(A, W, bias=None, residual=None, act="none", out=None, out_dtype=None):
    """Y = act(A @ W + bias) + residual in one kernel.

    A [M,K], W [K,N], bias [N], residual [M,N]; fp16 or bf16, contiguous, on one
    GPU.  ``out_dtype`` may be torch.float32.  ``out`` may be ``residual``
    (in-place update) when the output dtype is the input dtype.
    """
    torch = _torch()
    M, K = A.shape
    N = W.shape[1]
    _check(W, "W", A.dtype, (K, N), A.device)
    _check(bias, "bias", A.dtype, (N,), A.device)
    _check(residual, "residual", A.dtype, (M, N), A.device)
    code = _dtype_code(A, out_dtype)
    Y = _out(out, (M, N), torch.float32 if code & OUT_F32 else A.dtype, A.device)
    rc = lib().fuse_gemm_epilogue(_ptr(A), _ptr(W), _ptr(bias), _ptr(residual), _ptr(Y),
                                  M, N, K, _act(act), code, _stream(A.device))
    if rc != 0:
        raise FuseError(rc, "fuse_gemm_epilogue")
    return Y


def rmsnorm_gemm(X, gamma, W, eps=1e-6, bias=None, act="none", out=None, out_dtype=None, noalloc=False):
    """Y = act(RMSNorm_{gamma,eps}(X) @ W + bias); the normalised X stays on chip.

    ``noalloc=True`` calls fuse_rmsnorm_gemm_noalloc (no device allocation by
    the library; pass ``out`` too, so that nothing is allocated here either)."""
    torch = _torch()
    M, K = X.shape
    N = W.shape[1]
    _check(gamma, "gamma", X.dtype, (K,), X.device)
    _check(W, "W", X.dtype, (K, N), X.device)
    _check(bias, "bias", X.dtype, (N,), X.device)
    code = _dtype_code(X, out_dtype)
    Y = _out(out, (M, N), torch.float32 if code & OUT_F32 else X.dtype, X.device)
    fn = lib().fuse_rmsnorm_gemm_noalloc if noalloc else lib().fuse_rmsnorm_gemm
    rc = fn(_ptr(X), _ptr(gamma), float(eps), _ptr(W), _ptr(bias), _ptr(Y), M, N, K, _act(act), code,
            _stream(X.device))
    if rc != 0:
        raise FuseError(rc, "fuse_rmsnorm_gemm_noalloc" if noalloc else "fuse_rmsnorm_gemm")
    return Y


def layernorm_gemm(X, gamma, W, eps=1e-5, beta=None, bias=None, act="none", out=None, out_dtype=None):
    """Y = act(LayerNorm_{gamma,beta,eps}(X) @ W + bias); the normalised X stays on chip."""
    torch = _torch()
    M, K = X.shape
    N = W.shape[1]
    _check(gamma, "gamma", X.dtype, (K,), X.device)
    _check(beta, "beta", X.dtype, (K,), X.device)
    _check(W, "W", X.dtype, (K, N), X.device)
    _check(bias, "bias", X.dtype, (N,), X.device)
    code = _dtype_code(X, out_dtype)
    Y = _out(out, (M, N), torch.float32 if code & OUT_F32 else X.dtype, X.device)
    rc = lib().fuse_layernorm_gemm(_ptr(X), _ptr(gamma), _ptr(beta), float(eps), _ptr(W), _ptr(bias), _ptr(Y),
                                   M, N, K, _act(act), code, _stream(X.device))
    if rc != 0:
        raise FuseError(rc, "fuse_layernorm_gemm")
    return Y


def gemm_prologue_bias(A, abias, W, bias=None, residual=None, act="none", out=None, out_dtype=None):
    """Y = act((A + abias) @ W + bias) + residual; abias [K] is added to A inside the reduction."""
    torch = _torch()
    M, K = A.shape
    N = W.shape[1]
    _check(abias, "abias", A.dtype, (K,), A.device)
    _check(W, "W", A.dtype, (K, N), A.device)
    _check(bias, "bias", A.dtype, (N,), A.device)
    _check(residual, "residual", A.dtype, (M, N), A.device)
    code = _dtype_code(A, out_dtype)
    Y = _out(out, (M, N), torch.float32 if code & OUT_F32 else A.dtype, A.device)
    rc = lib().fuse_gemm_prologue_bias(_ptr(A), _ptr(abias), _ptr(W), _ptr(bias), _ptr(residual), _ptr(Y),
                                       M, N, K, _act(act), code, _stream(A.device))
    if rc != 0:
        raise FuseError(rc, "fuse_gemm_prologue_bias")
    return Y


def rmsnorm_gemm_swiglu(X, gamma, Wg, Wu, eps=1e-6, out=None, out_dtype=None):
    """H = SiLU(Xhat @ Wg) * (Xhat @ Wu), Xhat = RMSNorm_{gamma,eps}(X), in one kernel."""
    torch = _torch()
    M, K = X.shape
    F = Wg.shape[1]
    _check(gamma, "gamma", X.dtype, (K,), X.device)
    _check(Wg, "Wg", X.dtype, (K, F), X.device)
    _check(Wu, "Wu", X.dtype, (K, F), X.device)
    code = _dtype_code(X, out_dtype)
    H = _out(out, (M, F), torch.float32 if code & OUT_F32 else X.dtype, X.device)
    rc = lib().fuse_rmsnorm_gemm_swiglu(_ptr(X), _ptr(gamma), float(eps), _ptr(Wg), _ptr(Wu), _ptr(H),
                                        M, F, K, code, _stream(X.device))
    if rc != 0:
        raise FuseError(rc, "fuse_rmsnorm_gemm_swiglu")
    return H


def swiglu_ffn(X, gamma, Wg, Wu, Wd, bias_d, eps=1e-6, out_dtype=None, H=None, out=None):
    """SwiGLU FFN block as two fused kernels: H = rmsnorm_gemm_swiglu(X), Y = H @ Wd + bias_d + X."""
    H = rmsnorm_gemm_swiglu(X, gamma, Wg, Wu, eps=eps, out=H)
    return gemm_epilogue(H, Wd, bias_d, X, "none", out=out, out_dtype=out_dtype)


def plan_name(op: int, M: int, N: int, K: int, dtype: int = F16) -> str:
    return lib().fuse_plan_name(op, M, N, K, dtype).decode()


def workspace_bytes(op: int, M: int, N: int, K: int, dtype: int = F16) -> int:
    """Bytes of split-K workspace a call would use (0: its plan does not split K)."""
    n = lib().fuse_workspace_bytes(op, M, N, K, dtype)
    if n < 0:
        raise ValueError("invalid op, dtype or shape")
    return n


def set_plan(name):
    """Force a tile plan by name, "<plan>" or "<plan>:k<S>" (None or "" restores the automatic
    choice); it applies to the calls it fits, the automatic choice to the others."""
    rc = lib().fuse_set_plan(None if name is None else name.encode())
    if rc != 0:
        raise FuseError(rc, "fuse_set_plan")
