"""RMSNorm -> Linear (and the SwiGLU gate/up pair) on rows at the edges of
the number range, compared with the fp64 oracle over the whole output (needs
an MI355X).

The normalised activation is x * r * gamma with r = 1 / sqrt(mean(x^2) + eps)
("LLMBoost", section 3; deplodock post, RMSNorm loop nest), and it is finite
and of unit scale for every finite row.  The kernels' fast path forms
round(x * gamma) and applies r afterwards, which leaves the fp16 range when
|x * gamma| >= 65520 and magnifies subnormal rounding when mean(x^2) + eps is
tiny; those tiles must be recomputed exactly.  Each tile plan is forced in
turn, with rows laid out so that the first 256 rows hold only rows the fast
path serves (unit rows and rows at 2^-14 scale with eps = 0) and the next 256
rows mix in rows it must hand over (a maximum |x| of 64000 with gamma > 1,
rows at 2^-17 scale with eps = 0; in bf16 rows at 2^64 and 2^-70 scale).
"""
import numpy as np
import pytest

import gemm_epilogue_fuse_amd as lf
import oracle
import synth
from parity_util import DUAL_PLANS, PLANS, assert_close, dev_t, fitk, say, to64

pytestmark = pytest.mark.gpu

M, N = 520, 136


def row_layout(dtype):
    """Per-row (kind, value): ("rms", s) scales a unit-normal row to RMS s,
    ("max", v) scales it so its largest |x| is v."""
    if dtype == synth.F16:
        fast = [("rms", 1.0), ("rms", 2.0 ** -14), ("rms", 3.0)]
        edge = [("max", 64000.0), ("rms", 2.0 ** -17), ("rms", 1.0), ("max", 60000.0)]
    else:
        fast = [("rms", 1.0), ("rms", 2.0 ** -40), ("rms", 2.0 ** 40)]
        edge = [("rms", 2.0 ** 64), ("rms", 2.0 ** -70), ("rms", 1.0), ("rms", 2.0 ** 70)]
    rows = [fast[m % len(fast)] for m in range(256)]
    rows += [edge[m % len(edge)] for m in range(256)]
    rows += [("rms", 1.0)] * (M - 512)
    return rows


def range_inputs(K, F, dtype, seed, w_std=None):
    """X rows at the scales of row_layout, gamma = 1.1 + N(0, 0.05) (above 1, so the
    64000-rows overflow fp16 when multiplied by gamma), W and Wu ~ N(0, w_std)
    (default 1/sqrt(K)), bias ~ N(0, 0.1)."""
    g = synth.generator(seed)
    Z = synth.normal(g, (M, K), 1.0)
    X = np.empty_like(Z)
    for m, (kind, v) in enumerate(row_layout(dtype)):
        z = Z[m]
        X[m] = z * (v / np.sqrt(np.mean(z * z)) if kind == "rms" else v / np.max(np.abs(z)))
    gamma = synth.normal(g, (K,), 0.05, 1.1)
    w_std = 1.0 / np.sqrt(K) if w_std is None else w_std
    W = synth.normal(g, (K, F), w_std)
    Wu = synth.normal(g, (K, F), w_std)
    b = synth.normal(g, (F,), 0.1)
    bits = {k: synth.to_bits(v, dtype) for k, v in (("X", X), ("gamma", gamma), ("W", W), ("Wu", Wu),
                                                      ("bias", b))}
    assert np.all(np.isfinite(synth.widen(bits["X"], dtype)))
    return bits


@pytest.fixture(params=PLANS)
def plan(request):
    lf.set_plan(request.param)
    yield request.param
    lf.set_plan(None)


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_rmsnorm_gemm_row_range(plan, dtype):
    import torch
    K = fitk(plan, 520)
    assert lf.plan_name(1, M, N, K) == plan
    d = range_inputs(K, N, dtype, seed=41)
    t = {k: dev_t(v, dtype) for k, v in d.items()}
    x = {k: synth.widen(v, dtype) for k, v in d.items()}
    for eps in (1e-6, 0.0):
        eps32 = float(np.float32(eps))
        say("rms-range", plan, dtype, M, K, N, "eps", eps)
        want = oracle.rmsnorm_gemm(x["X"], x["gamma"], eps32, x["W"][:, :N], x["bias"][:N], "gelu_tanh")
        assert np.all(np.isfinite(want))
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
        W = t["W"][:, :N].contiguous()
        got = to64(lf.rmsnorm_gemm(t["X"], t["gamma"], W, eps, t["bias"][:N].contiguous(), "gelu_tanh",
                                   out=out, out_dtype=torch.float32))
        assert_close(got, want, "f32out eps=%g" % eps)
        assert_close(got[:256], want[:256], "fast-path rows eps=%g" % eps)
        if dtype == synth.F16:
            got16 = to64(lf.rmsnorm_gemm(t["X"], t["gamma"], W, eps, t["bias"][:N].contiguous(), "gelu_tanh"))
            assert_close(got16, want, "f16out eps=%g" % eps)


@pytest.fixture(params=DUAL_PLANS)
def dual_plan(request):
    lf.set_plan(request.param)
    yield request.param
    lf.set_plan(None)


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_swiglu_row_range(dual_plan, dtype):
    import torch
    K, F = 512, 136
    d = range_inputs(K, F, dtype, seed=42, w_std=1.0 / 64.0)
    t = {k: dev_t(v, dtype) for k, v in d.items()}
    x = {k: synth.widen(v, dtype) for k, v in d.items()}
    for eps in (1e-6, 0.0):
        eps32 = float(np.float32(eps))
        say("swiglu-range", dual_plan or "auto", lf.plan_name(2, M, F, K, lf.BF16 if dtype == synth.BF16 else lf.F16),
            dtype, "eps", eps)
        want = oracle.rmsnorm_swiglu(x["X"], x["gamma"], eps32, x["W"], x["Wu"])
        out = torch.full((M, F), float("nan"), dtype=torch.float32, device="cuda:0")
        got = to64(lf.rmsnorm_gemm_swiglu(t["X"], t["gamma"], t["W"], t["Wu"], eps, out=out,
                                          out_dtype=torch.float32))
        assert_close(got, want, "H f32out eps=%g" % eps)
