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


# Tile plans, and DMA plans with a forced split-K count (":k<S>"): the
# splits of a tile are reduced in a fixed order by the last one to finish.
PLANS = ["dma_256x256x32_s4", "dma_128x128x64_s4", "reg_256x256x64", "reg_128x128x64",
         "dma_128x128x64_s4:k3", "dma_128x128x64_s4:k2", "dma_256x256x32_s4_w8",
         "dma_128x128x64_s4_g2", "dma_128x128x64_s4_g2:k2", "dma_128x128x64_s4_g2:k3",
         "dma_128x128x32_s8_g2", "dma_128x128x32_s8_g2:k2", "dec_32x64", "dec_32x64:k3",
         "strip_16x16", "strip_32x16", "dma_256x128x32_s6_w8", "dma_256x128x32_s6_w8:k3",
         "dma_256x128x64_s3_w8", "dma_256x128x64_s3_w8:k2", "wstrip_16x16", "wstrip_32x16",
         "dma_64x128x64_s4_g2", "dma_64x128x64_s4_g2:k3", "dma_256x128x64_s3", "dma_256x128x64_s3:k2"]
# Gate/up dual-GEMM plans ("" = automatic choice); a forced DMA plan applies where K
# is a multiple of its K step, the automatic choice elsewhere.
DUAL_PLANS = ["", "dma_dual_256x128x32_s4", "reg_dual_256x128x64"]


def fitk(plan, K):
    """DMA and small-M plans need K % 64 == 0 (strips K % 128, whole strips K % 256): round K up for them
    (M and N stay ragged);
    split plans get at least 3 K steps per split."""
    if not plan.startswith(("dma", "dec", "strip", "wstrip")):
        return K
    step = 256 if plan.startswith("wstrip") else 128 if plan.startswith("strip") else 64
    K = -(-K // step) * step
    if plan.startswith("dec") and ":k" not in plan:
        K = min(K, 512)  # one K chunk: at most 8 steps of 64
    if ":k" in plan:
        K = max(K, 64 * 3 * int(plan.split(":k")[1]))
    return K


def base(plan):
    return plan.split(":")[0]
