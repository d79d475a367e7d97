"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds no arithmetic of the operators themselves: it only draws
random numbers, rounds them to the 16-bit storage formats, and widens stored
16-bit values back to float64.  Both the HIP path and the oracle receive the
same bits from here.

Recipe (the workloads of the fused-GEMM and RMSNorm->Linear pages, as sized in
the operator's configuration list):

1. ``numpy.random.Generator(PCG64(seed))``, seed 0 unless stated.
2. float64 standard normals, drawn tensor by tensor in the order the workload
   names them, scaled by the stated standard deviation ("N(0, s)" means
   standard deviation s) and shifted by the stated mean (gamma = 1 + N(0, 0.1)).
3. Rounded to the storage dtype with round-to-nearest-even: fp16 directly from
   float64 (numpy's correctly rounded cast); bf16 from float64 via float32,
   each step round-to-nearest-even.
"""
from __future__ import annotations

from collections import OrderedDict

import numpy as np

F16 = "f16"
BF16 = "bf16"


def generator(seed: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bits(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to fp16/bf16 (nearest-even); return raw uint16 bits."""
    x64 = np.asarray(x64, dtype=np.float64)
    if dtype == F16:
        return x64.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = x64.astype(np.float32).view(np.uint32).astype(np.uint64)
        is_nan = np.isnan(x64)
        rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        out = rounded.astype(np.uint16)
        if is_nan.any():
            out = np.where(is_nan, np.uint16(0x7FC0), out)
        return out
    raise ValueError(dtype)


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored fp16/bf16 bits."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def to_torch(bits: np.ndarray, dtype: str, device="cpu"):
    """Torch tensor holding exactly these 16-bit values."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.float16 if dtype == F16 else torch.bfloat16)
    return t.to(device)


def normal(g: np.random.Generator, shape, std: float, mean: float = 0.0) -> np.ndarray:
    return g.standard_normal(size=shape) * std + mean


def _pack(fields, dtype):
    return OrderedDict((k, to_bits(v, dtype)) for k, v in fields)


def gemm_bias_gelu_small(seed: int = 0, dtype: str = F16):
    """64x256x256 GEMM + bias + GeLU: A ~ N(0,1), W ~ N(0, 1/sqrt(256)), bias ~ N(0, 0.1)."""
    g = generator(seed)
    M, K, N = 64, 256, 256
    A = normal(g, (M, K), 1.0)
    W = normal(g, (K, N), 1.0 / np.sqrt(K))
    b = normal(g, (N,), 0.1)
    return _pack([("A", A), ("W", W), ("bias", b)], dtype)


def rmsnorm_linear(M: int = 512, D: int = 4096, N: int = 4096, seed: int = 0, dtype: str = F16,
                   w_std: float = None, order=("X", "gamma", "W")):
    """RMSNorm -> Linear inputs: X ~ N(0,1), gamma = 1 + N(0,0.1), W ~ N(0, w_std).

    ``order`` is the draw order; the prefill workload names X, gamma, W; the
    decode sweep names W, X, gamma.
    """
    g = generator(seed)
    if w_std is None:
        w_std = 1.0 / np.sqrt(D)
    shapes = {"X": ((M, D), 1.0, 0.0), "gamma": ((D,), 0.1, 1.0), "W": ((D, N), w_std, 0.0)}
    drawn = {}
    for name in order:
        shp, std, mean = shapes[name]
        drawn[name] = normal(g, shp, std, mean)
    return _pack([(k, drawn[k]) for k in ("X", "gamma", "W")], dtype)


def gemm_epilogue_sweep(M: int, N: int = 4096, K: int = 4096, seed: int = 0, dtype: str = F16,
                        residual: bool = False):
    """A ~ N(0,1), W ~ N(0,1/64), bias ~ N(0,0.1), optionally R ~ N(0,1) [M,N]."""
    g = generator(seed)
    fields = [("A", normal(g, (M, K), 1.0)), ("W", normal(g, (K, N), 1.0 / 64.0)),
              ("bias", normal(g, (N,), 0.1))]
    if residual:
        fields.append(("R", normal(g, (M, N), 1.0)))
    return _pack(fields, dtype)


def swiglu_ffn(M: int = 2048, D: int = 4096, F: int = 11008, seed: int = 0, dtype: str = BF16):
    """X ~ N(0,1), gamma = 1+N(0,0.1), Wg, Wu ~ N(0,1/64) [D,F], Wd ~ N(0,1/105) [F,D], bias ~ N(0,0.1)."""
    g = generator(seed)
    X = normal(g, (M, D), 1.0)
    gamma = normal(g, (D,), 0.1, 1.0)
    Wg = normal(g, (D, F), 1.0 / 64.0)
    Wu = normal(g, (D, F), 1.0 / 64.0)
    Wd = normal(g, (F, D), 1.0 / 105.0)
    b = normal(g, (D,), 0.1)
    return _pack([("X", X), ("gamma", gamma), ("Wg", Wg), ("Wu", Wu), ("Wd", Wd), ("bias", b)], dtype)


def decode_rmsnorm_linear(B: int, D: int, seed: int = 0, dtype: str = F16):
    """Decode-shaped RMSNorm -> Linear: W[D,D] ~ N(0,1/sqrt(D)), X[B,D] ~ N(0,1), gamma = 1+N(0,0.1)."""
    return rmsnorm_linear(M=B, D=D, N=D, seed=seed, dtype=dtype, w_std=1.0 / np.sqrt(D),
                          order=("W", "X", "gamma"))
