"""fp64 CPU oracle for the fused GEMM + epilogue and RMSNorm -> Linear operator.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``gemm_epilogue_fuse_amd``) never imports it, and this package imports nothing
from the product path: the two share no code, headers, tables or helpers.

The arithmetic lives in ``oracle.c`` (plain C, double precision, no rounding
between steps).  This module builds it with gcc if needed and exposes numpy
wrappers.  ``brute.py`` next to it is an independent pure-Python version for
tiny shapes.

Parts and the passages they follow (page title, section):

* ``gemm_epilogue``  -- "llm-fusion-compiler", pattern table and usage example
  (gemm, then bias, then activation; residual pattern); deplodock post, Tensor
  IR (matmul as broadcast multiply summed over the shared axis).
* ``act``            -- "llm-fusion-compiler", pattern table and results (GeLU
  in tanh form, deviation 0.000473 from exact GeLU); SiLU = z*sigmoid(z)
  (standard, the pages do not define it); ReLU = max(0, z).
* ``rms_factor`` / ``rmsnorm`` -- deplodock post, RMSNorm loop nest (sum of
  squares, times 1/n, plus eps, rsqrt, times x, times weight); "LLMBoost",
  section 3 (rsqrt(sum_sq / d_in + eps)).
* ``rmsnorm_gemm``   -- "LLMBoost", problem statement (RMSNorm feeding the next
  Linear) composed with ``gemm_epilogue``.
* ``rmsnorm_swiglu`` / ``swiglu_ffn`` -- "llm-fusion-compiler", FFN block
  (SwiGLU style: three GEMMs, activation, elementwise product, bias,
  residual).
* ``layernorm`` / ``layernorm_gemm`` -- "llm-fusion-compiler", pattern table
  (layernorm_gemm); the page names LayerNorm without printing it, so this is
  the standard definition (mean, biased variance, eps inside the root, affine
  gamma and beta).
* ``prologue_bias_gemm`` -- deplodock post, Loop IR worked example
  relu((x + bias) @ w): the bias is added to x inside the reduce, before the
  products, and the activation follows the reduction.

Every function here is pinned by ``tests/test_oracle_pins.py`` against values
that do not come from the oracle itself (identity and permutation weights,
integer data against integer matmul, numpy/torch library special cases, closed
forms, the pages' GeLU deviation figure, and brute force on tiny shapes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ACT_NONE, ACT_RELU, ACT_GELU_TANH, ACT_SILU = 0, 1, 2, 3
ACT_CODES = {"none": ACT_NONE, "relu": ACT_RELU, "gelu_tanh": ACT_GELU_TANH, "silu": ACT_SILU}

_lib = None


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oracle_act.restype = ctypes.c_double
        lib.oracle_act.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.oracle_act_vec.restype = None
        lib.oracle_act_vec.argtypes = [dp, dp, i64, ctypes.c_int]
        lib.oracle_gemm_epilogue.restype = ctypes.c_int
        lib.oracle_gemm_epilogue.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, ctypes.c_int]
        lib.oracle_rms_factor.restype = None
        lib.oracle_rms_factor.argtypes = [dp, dp, i64, i64, ctypes.c_double]
        lib.oracle_rmsnorm.restype = None
        lib.oracle_rmsnorm.argtypes = [dp, dp, ctypes.c_double, dp, i64, i64]
        lib.oracle_rmsnorm_gemm.restype = ctypes.c_int
        lib.oracle_rmsnorm_gemm.argtypes = [dp, dp, ctypes.c_double, dp, dp, dp, i64, i64, i64, ctypes.c_int]
        lib.oracle_rmsnorm_swiglu.restype = ctypes.c_int
        lib.oracle_rmsnorm_swiglu.argtypes = [dp, dp, ctypes.c_double, dp, dp, dp, i64, i64, i64]
        lib.oracle_layernorm.restype = None
        lib.oracle_layernorm.argtypes = [dp, dp, dp, ctypes.c_double, dp, i64, i64]
        lib.oracle_layernorm_gemm.restype = ctypes.c_int
        lib.oracle_layernorm_gemm.argtypes = [dp, dp, dp, ctypes.c_double, dp, dp, dp, i64, i64, i64, ctypes.c_int]
        lib.oracle_prologue_bias_gemm.restype = ctypes.c_int
        lib.oracle_prologue_bias_gemm.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64, i64, ctypes.c_int]
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _act_code(act) -> int:
    if isinstance(act, str):
        return ACT_CODES[act]
    return int(act)


def act(z, act_kind) -> np.ndarray:
    """Elementwise activation in fp64."""
    z = _f64(z)
    out = np.empty_like(z)
    _load().oracle_act_vec(_ptr(z.reshape(-1)), _ptr(out.reshape(-1)), z.size, _act_code(act_kind))
    return out


def gemm_epilogue(A, W, bias=None, residual=None, act_kind="none") -> np.ndarray:
    """Y = act(A @ W + bias) + residual, all in fp64.  A [M,K], W [K,N]."""
    A, W, bias, residual = _f64(A), _f64(W), _f64(bias), _f64(residual)
    M, K = A.shape
    K2, N = W.shape
    assert K == K2, "A and W disagree on K"
    if bias is not None:
        assert bias.shape == (N,)
    if residual is not None:
        assert residual.shape == (M, N)
    Y = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_epilogue(_ptr(A), _ptr(W), _ptr(bias), _ptr(residual), _ptr(Y),
                                      M, N, K, _act_code(act_kind))
    if rc != 0:
        raise ValueError("oracle_gemm_epilogue failed (%d)" % rc)
    return Y


def rms_factor(X, eps) -> np.ndarray:
    """r[m] = 1/sqrt(mean_k x[m,k]^2 + eps)."""
    X = _f64(X)
    M, K = X.shape
    r = np.empty((M,), dtype=np.float64)
    _load().oracle_rms_factor(_ptr(X), _ptr(r), M, K, float(eps))
    return r


def rmsnorm(X, gamma, eps) -> np.ndarray:
    """Xhat = X * r[:,None] * gamma[None,:] in fp64."""
    X, gamma = _f64(X), _f64(gamma)
    M, K = X.shape
    assert gamma.shape == (K,)
    out = np.empty_like(X)
    _load().oracle_rmsnorm(_ptr(X), _ptr(gamma), float(eps), _ptr(out), M, K)
    return out


def rmsnorm_gemm(X, gamma, eps, W, bias=None, act_kind="none") -> np.ndarray:
    """Y = act(RMSNorm(X) @ W + bias) in fp64."""
    X, gamma, W, bias = _f64(X), _f64(gamma), _f64(W), _f64(bias)
    M, K = X.shape
    K2, N = W.shape
    assert K == K2 and gamma.shape == (K,)
    Y = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_rmsnorm_gemm(_ptr(X), _ptr(gamma), float(eps), _ptr(W), _ptr(bias), _ptr(Y),
                                     M, N, K, _act_code(act_kind))
    if rc != 0:
        raise ValueError("oracle_rmsnorm_gemm failed (%d)" % rc)
    return Y


def rmsnorm_swiglu(X, gamma, eps, Wg, Wu) -> np.ndarray:
    """H = SiLU(RMSNorm(X) @ Wg) * (RMSNorm(X) @ Wu) in fp64."""
    X, gamma, Wg, Wu = _f64(X), _f64(gamma), _f64(Wg), _f64(Wu)
    M, K = X.shape
    K2, F = Wg.shape
    assert K == K2 and Wu.shape == (K, F) and gamma.shape == (K,)
    H = np.empty((M, F), dtype=np.float64)
    rc = _load().oracle_rmsnorm_swiglu(_ptr(X), _ptr(gamma), float(eps), _ptr(Wg), _ptr(Wu), _ptr(H), M, F, K)
    if rc != 0:
        raise ValueError("oracle_rmsnorm_swiglu failed (%d)" % rc)
    return H


def swiglu_ffn(X, gamma, eps, Wg, Wu, Wd, bias_d) -> np.ndarray:
    """Whole SwiGLU FFN block: Y = H @ Wd + bias_d + X, H from ``rmsnorm_swiglu``."""
    H = rmsnorm_swiglu(X, gamma, eps, Wg, Wu)
    return gemm_epilogue(H, Wd, bias_d, X, "none")


def layernorm(X, gamma, eps, beta=None) -> np.ndarray:
    """(X - mean) / sqrt(biased variance + eps) * gamma + beta over the last axis, in fp64."""
    X, gamma, beta = _f64(X), _f64(gamma), _f64(beta)
    M, K = X.shape
    assert gamma.shape == (K,) and (beta is None or beta.shape == (K,))
    out = np.empty_like(X)
    _load().oracle_layernorm(_ptr(X), _ptr(gamma), _ptr(beta), float(eps), _ptr(out), M, K)
    return out


def layernorm_gemm(X, gamma, eps, W, beta=None, bias=None, act_kind="none") -> np.ndarray:
    """Y = act(LayerNorm(X) @ W + bias) in fp64."""
    X, gamma, beta, W, bias = _f64(X), _f64(gamma), _f64(beta), _f64(W), _f64(bias)
    M, K = X.shape
    K2, N = W.shape
    assert K == K2 and gamma.shape == (K,)
    Y = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_layernorm_gemm(_ptr(X), _ptr(gamma), _ptr(beta), float(eps), _ptr(W), _ptr(bias),
                                       _ptr(Y), M, N, K, _act_code(act_kind))
    if rc != 0:
        raise ValueError("oracle_layernorm_gemm failed (%d)" % rc)
    return Y


def prologue_bias_gemm(A, abias, W, bias=None, residual=None, act_kind="none") -> np.ndarray:
    """Y = act((A + abias) @ W + bias) + residual in fp64; abias [K] is added to every row of A."""
    A, abias, W, bias, residual = _f64(A), _f64(abias), _f64(W), _f64(bias), _f64(residual)
    M, K = A.shape
    K2, N = W.shape
    assert K == K2 and abias.shape == (K,)
    Y = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_prologue_bias_gemm(_ptr(A), _ptr(abias), _ptr(W), _ptr(bias), _ptr(residual), _ptr(Y),
                                           M, N, K, _act_code(act_kind))
    if rc != 0:
        raise ValueError("oracle_prologue_bias_gemm failed (%d)" % rc)
    return Y
