"""Pure-Python brute force of the same operators, for tiny shapes only.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Written separately from
``oracle.c`` (plain nested lists, ``math`` functions) so that the two can pin
each other on tiny inputs: a dropped term, a wrong index or a transposed
operand in either one shows up as a mismatch.

Definitions followed (page title, section): "llm-fusion-compiler" pattern
table (gemm -> bias -> activation, residual add after), deplodock post RMSNorm
loop nest, "LLMBoost" section 3 (per-row rsqrt of mean square plus eps),
"llm-fusion-compiler" pattern table (layernorm_gemm: LayerNorm with mean,
biased variance, eps inside the root, gamma and beta), deplodock post Loop IR
example (relu((x + bias) @ w): bias added to x before the reduction).
"""
from __future__ import annotations

import math


def act(z: float, kind: str) -> float:
    if kind == "none":
        return z
    if kind == "relu":
        return z if z > 0.0 else 0.0
    if kind == "gelu_tanh":
        c = math.sqrt(2.0 / math.pi)
        return 0.5 * z * (1.0 + math.tanh(c * (z + 0.044715 * z ** 3)))
    if kind == "silu":
        # z * sigmoid(z), with sigmoid written in the overflow-free branch form
        if z >= 0:
            return z / (1.0 + math.exp(-z))
        e = math.exp(z)
        return z * e / (1.0 + e)
    raise ValueError(kind)


def matmul(A, W):
    M, K, N = len(A), len(W), len(W[0])
    out = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += A[i][k] * W[k][j]
            out[i][j] = s
    return out


def gemm_epilogue(A, W, bias=None, residual=None, kind="none"):
    C = matmul(A, W)
    M, N = len(C), len(C[0])
    Y = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            z = C[i][j] + (bias[j] if bias is not None else 0.0)
            Y[i][j] = act(z, kind) + (residual[i][j] if residual is not None else 0.0)
    return Y


def rmsnorm(X, gamma, eps):
    out = []
    for row in X:
        n = len(row)
        ms = sum(v * v for v in row) / n
        r = 1.0 / math.sqrt(ms + eps)
        out.append([row[k] * r * gamma[k] for k in range(n)])
    return out


def rmsnorm_gemm(X, gamma, eps, W, bias=None, kind="none"):
    return gemm_epilogue(rmsnorm(X, gamma, eps), W, bias, None, kind)


def rmsnorm_swiglu(X, gamma, eps, Wg, Wu):
    xh = rmsnorm(X, gamma, eps)
    G = matmul(xh, Wg)
    U = matmul(xh, Wu)
    return [[act(G[i][j], "silu") * U[i][j] for j in range(len(G[0]))] for i in range(len(G))]


def layernorm(X, gamma, eps, beta=None):
    out = []
    for row in X:
        n = len(row)
        mu = sum(row) / n
        var = sum((v - mu) * (v - mu) for v in row) / n
        r = 1.0 / math.sqrt(var + eps)
        out.append([(row[k] - mu) * r * gamma[k] + (beta[k] if beta is not None else 0.0) for k in range(n)])
    return out


def layernorm_gemm(X, gamma, eps, W, beta=None, bias=None, kind="none"):
    return gemm_epilogue(layernorm(X, gamma, eps, beta), W, bias, None, kind)


def prologue_bias_gemm(A, abias, W, bias=None, residual=None, kind="none"):
    shifted = [[row[k] + abias[k] for k in range(len(row))] for row in A]
    return gemm_epilogue(shifted, W, bias, residual, kind)
