"""Small torch modules for the graph-level fusion tests: the transformer
pieces the fusion patterns target, written the way model code writes them."""
import torch
import torch.nn as nn
import torch.nn.functional as F


class RmsLinearGelu(nn.Module):
    """RMSNorm -> Linear (bias) -> GeLU(tanh)."""

    def __init__(self, D=64, N=48):
        super().__init__()
        self.norm = nn.RMSNorm(D, eps=1e-6)
        self.proj = nn.Linear(D, N)
        self.act = nn.GELU(approximate="tanh")

    def forward(self, x):
        return self.act(self.proj(self.norm(x)))


class DecomposedRmsNorm(nn.Module):
    """RMSNorm written out (x * rsqrt(mean(x^2) + eps) * weight, with casts)."""

    def __init__(self, D, eps=1e-6):
        super().__init__()
        self.weight = nn.Parameter(1.0 + 0.1 * torch.randn(D))
        self.eps = eps

    def forward(self, h):
        dt = h.dtype
        h = h.to(torch.float32)
        var = h.pow(2).mean(-1, keepdim=True)
        h = h * torch.rsqrt(var + self.eps)
        return self.weight * h.to(dt)


class DecomposedRmsQProj(nn.Module):
    def __init__(self, D=64, N=64):
        super().__init__()
        self.norm = DecomposedRmsNorm(D)
        self.q = nn.Linear(D, N, bias=False)

    def forward(self, x):
        return self.q(self.norm(x))


class SharedNormQKV(nn.Module):
    """One RMSNorm output read by three projections: fusing the norm into any
    one would recompute or buffer it for the others."""

    def __init__(self, D=64):
        super().__init__()
        self.norm = nn.RMSNorm(D, eps=1e-6)
        self.q, self.k, self.v = (nn.Linear(D, D, bias=True) for _ in range(3))

    def forward(self, x):
        h = self.norm(x)
        return self.q(h), self.k(h), self.v(h)


class SwiGluMlp(nn.Module):
    """RMSNorm -> gate / up -> SiLU(gate) * up -> down (+ residual)."""

    def __init__(self, D=64, F_=96):
        super().__init__()
        self.norm = nn.RMSNorm(D, eps=1e-6)
        self.gate = nn.Linear(D, F_, bias=False)
        self.up = nn.Linear(D, F_, bias=False)
        self.down = nn.Linear(F_, D, bias=True)

    def forward(self, x):
        h = self.norm(x)
        return self.down(F.silu(self.gate(h)) * self.up(h)) + x


class LnLinearRelu(nn.Module):
    def __init__(self, D=64, N=40):
        super().__init__()
        self.ln = nn.LayerNorm(D, eps=1e-5)
        self.fc = nn.Linear(D, N)

    def forward(self, x):
        return F.relu(self.fc(self.ln(x)))


class PrologueBias(nn.Module):
    """The deplodock post's relu((x + bias) @ w)."""

    def __init__(self, K=64, N=16):
        super().__init__()
        self.bias = nn.Parameter(torch.randn(K))
        self.w = nn.Parameter(torch.randn(K, N) / 8.0)

    def forward(self, x):
        return torch.relu(torch.matmul(x + self.bias, self.w))


class MatmulBiasActResidual(nn.Module):
    """x @ W + b -> SiLU -> + r, with an exact GeLU branch the matcher must leave alone."""

    def __init__(self, K=64, N=48):
        super().__init__()
        self.w = nn.Parameter(torch.randn(K, N) / 8.0)
        self.b = nn.Parameter(0.1 * torch.randn(N))
        self.w2 = nn.Parameter(torch.randn(K, N) / 8.0)
        self.b2 = nn.Parameter(0.1 * torch.randn(N))

    def forward(self, x, r):
        y = F.silu(torch.matmul(x, self.w) + self.b) + r
        z = F.gelu(torch.matmul(x, self.w2) + self.b2)  # exact GeLU: only matmul + bias fuse
        return y, z
