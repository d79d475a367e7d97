"""Helpers shared by the GPU parity tests: device tensors from synthetic bits,
error metrics against the fp64 oracle, and the tolerance of the operator
(max_abs_err <= 1.5e-2, mean_abs_err <= 1.5e-3 for fp16/bf16 inputs with fp32
accumulation)."""
import sys

import numpy as np

import synth

MAX_ABS_TOL = 1.5e-2
MEAN_ABS_TOL = 1.5e-3
EPS = 1e-6
EPS32 = float(np.float32(EPS))


def say(*a):
    """Name the case before a GPU step, flushed, so a fault still leaves a trace."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev_t(bits, dtype):
    return synth.to_torch(bits, dtype, "cuda:0")


def to64(t):
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def errors(got, want):
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    return float(d.max()), float(d.mean())


def assert_close(got, want, what=""):
    assert np.all(np.isfinite(got)), "non-finite output %s" % what
    mx, mean = errors(got, want)
    say("  %s max_abs_err=%.3e mean_abs_err=%.3e" % (what, mx, mean))
    assert mx <= MAX_ABS_TOL, "%s: max_abs_err %.3e > %.1e" % (what, mx, MAX_ABS_TOL)
    assert mean <= MEAN_ABS_TOL, "%s: mean_abs_err %.3e > %.1e" % (what, mean, MEAN_ABS_TOL)
    return mx, mean


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def sample_rows(M, n, seed=0):
    """Rows checked at full size: first, last, and a seeded spread in between."""
    if M <= n:
        return np.arange(M)
    g = np.random.Generator(np.random.PCG64(seed + 7919))
    mid = g.choice(np.arange(1, M - 1), size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, M - 1], mid]))
