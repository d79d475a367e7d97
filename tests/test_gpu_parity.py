"""Parity of the HIP path against the fp64 oracle on seeded inputs (needs an
MI355X).

Small and ragged shapes are compared element by element over the whole
output, with every tile plan forced in turn; the workloads at their full
sizes run in the automatic plan (the one the bench times) and are compared
with the oracle over their whole output, written into NaN-filled buffers.
Tolerance: max_abs_err <= 1.5e-2 and mean_abs_err <= 1.5e-3.  bf16 runs are
checked with a float32 output against that bound (a bf16 output alone can be
off by half a bf16 ulp, 0.0156 at |y| in [4, 8), for any implementation), and
their bf16-output twin must be exactly the nearest-even rounding of that
float32 output.
"""
import numpy as np
import pytest

import gemm_epilogue_fuse_amd as lf
import oracle
import synth
from parity_util import DUAL_PLANS, EPS, EPS32, PLANS, assert_close, dev_t, fitk, say, to64

pytestmark = pytest.mark.gpu

ACTS = ["none", "relu", "gelu_tanh", "silu"]


def torch():
    import torch as t
    return t


def w64(d, dtype):
    return {k: synth.widen(v, dtype) for k, v in d.items()}


def check_bf16_output(got16, got32, want, what=""):
    """A bf16-output call must return exactly the nearest-even bf16 rounding of
    the float32-output call (same arithmetic, one final rounding); the float32
    output itself carries the oracle tolerance.  The raw errors of the bf16
    output are printed: they exceed the fp32-output tolerance by up to half a
    bf16 ulp, which no bf16-output kernel can avoid."""
    got16 = np.asarray(got16, dtype=np.float64)
    rounded = synth.widen(synth.to_bits(np.asarray(got32, dtype=np.float64), synth.BF16), synth.BF16)
    mism = np.sum(got16 != rounded)
    d = np.abs(got16 - want)
    say("  %s bf16-out raw max_abs_err=%.3e mean_abs_err=%.3e" % (what, d.max(), d.mean()))
    assert mism == 0, "bf16 output differs from RNE(fp32 output) at %d elements" % mism


@pytest.fixture(params=PLANS)
def plan(request):
    lf.set_plan(request.param)
    yield request.param
    lf.set_plan(None)


# --------------------------------------------------------------------------- small / ragged

@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("act", ACTS)
def test_gemm_epilogue_ragged(plan, dtype, act):
    T = torch()
    M, N, K = 300, 392, fitk(plan, 328)
    assert lf.plan_name(0, M, N, K) == plan
    say("gemm-ragged", plan, dtype, act, M, N, K)
    d = synth.gemm_epilogue_sweep(M, N, K, seed=21, dtype=dtype, residual=True)
    t = {k: dev_t(v, dtype) for k, v in d.items()}
    x = w64(d, dtype)
    for bias, res in ((True, False), (True, True), (False, False), (False, True)):
        want = oracle.gemm_epilogue(x["A"], x["W"], x["bias"] if bias else None, x["R"] if res else None, act)
        args = (t["A"], t["W"], t["bias"] if bias else None, t["R"] if res else None, act)
        out32 = to64(lf.gemm_epilogue(*args, out_dtype=T.float32))
        assert_close(out32, want, "%s bias=%d res=%d f32out" % (act, bias, res))
        out16 = to64(lf.gemm_epilogue(*args))
        if dtype == synth.F16:
            assert_close(out16, want, "%s bias=%d res=%d f16out" % (act, bias, res))
        else:
            check_bf16_output(out16, out32, want, act)


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("act", ACTS)
def test_rmsnorm_gemm_ragged(plan, dtype, act):
    T = torch()
    M, D, N = 260, fitk(plan, 520), 392
    assert lf.plan_name(1, M, N, D) == plan
    say("rms-ragged", plan, dtype, act, M, D, N)
    d = synth.rmsnorm_linear(M=M, D=D, N=N, seed=22, dtype=dtype)
    b = synth.to_bits(synth.generator(23).standard_normal(N) * 0.1, dtype)
    t = {k: dev_t(v, dtype) for k, v in d.items()}
    x = w64(d, dtype)
    bw = synth.widen(b, dtype)
    for bias in (False, True):
        want = oracle.rmsnorm_gemm(x["X"], x["gamma"], EPS32, x["W"], bw if bias else None, act)
        bt = dev_t(b, dtype) if bias else None
        out32 = to64(lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], EPS, bt, act, out_dtype=T.float32))
        assert_close(out32, want, "%s bias=%d f32out" % (act, bias))
        out16 = to64(lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], EPS, bt, act))
        if dtype == synth.F16:
            assert_close(out16, want, "%s bias=%d f16out" % (act, bias))
        else:
            check_bf16_output(out16, out32, want, act)


@pytest.fixture(params=DUAL_PLANS)
def dual_plan(request):
    lf.set_plan(request.param)
    yield request.param
    lf.set_plan(None)


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("M,F,K", [(300, 392, 328), (64, 136, 1000), (513, 264, 72), (300, 392, 320),
                                   (513, 264, 1024)])
def test_swiglu_ragged(dual_plan, dtype, M, F, K):
    T = torch()
    say("swiglu-ragged", dtype, M, F, K, lf.plan_name(2, M, F, K))
    d = synth.swiglu_ffn(M=M, D=K, F=F, seed=24, dtype=dtype)
    t = {k: dev_t(v, dtype) for k, v in d.items()}
    x = w64(d, dtype)
    want = oracle.rmsnorm_swiglu(x["X"], x["gamma"], EPS32, x["Wg"], x["Wu"])
    out32 = to64(lf.rmsnorm_gemm_swiglu(t["X"], t["gamma"], t["Wg"], t["Wu"], EPS, out_dtype=T.float32))
    assert_close(out32, want, "H f32out")
    out16 = to64(lf.rmsnorm_gemm_swiglu(t["X"], t["gamma"], t["Wg"], t["Wu"], EPS))
    if dtype == synth.F16:
        assert_close(out16, want, "H f16out")
    else:
        check_bf16_output(out16, out32, want, "H")


@pytest.mark.parametrize("wplan", ["wstrip_16x16", "wstrip_32x16"])
@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("M,N,K", [(1, 264, 1280), (5, 136, 2048), (17, 520, 3072), (32, 4104, 4096)])
def test_whole_strip_long_k(wplan, dtype, M, N, K):
    """The whole-strip kernels at 5..16 blocks of 32 k per wave (K = 1280..4096),
    where the padded block counts 8 and 16 are used; N % 16 == 8 leaves half of
    the last strip outside the output."""
    T = torch()
    lf.set_plan(wplan)
    try:
        assert lf.plan_name(1, M, N, K) == wplan
        say("whole-strip", wplan, dtype, M, N, K)
        d = synth.rmsnorm_linear(M=M, D=K, N=N, seed=25, dtype=dtype)
        g = synth.generator(26)
        b = synth.to_bits(g.standard_normal(N) * 0.1, dtype)
        R = synth.to_bits(g.standard_normal((M, N)), dtype)
        t = {k: dev_t(v, dtype) for k, v in d.items()}
        x = w64(d, dtype)
        want = oracle.rmsnorm_gemm(x["X"], x["gamma"], EPS32, x["W"], synth.widen(b, dtype), "gelu_tanh")
        out32 = to64(lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], EPS, dev_t(b, dtype), "gelu_tanh",
                                     out_dtype=T.float32))
        assert_close(out32, want, "rms gelu f32out")
        want = oracle.gemm_epilogue(x["X"], x["W"], synth.widen(b, dtype), synth.widen(R, dtype), "silu")
        out32 = to64(lf.gemm_epilogue(t["X"], t["W"], dev_t(b, dtype), dev_t(R, dtype), "silu", out_dtype=T.float32))
        assert_close(out32, want, "gemm silu residual f32out")
    finally:
        lf.set_plan(None)


# --------------------------------------------------------------------------- full sizes (automatic plan)
#
# Every workload at its full size, in the plan the bench times, compared with
# the oracle over the whole output.  Outputs are pre-filled with NaN, so an
# element no workgroup writes (a skipped tile, a dropped tail) fails the
# finiteness check, and one written twice with different values fails the
# comparison.

def nan_out(shape, dtype):
    T = torch()
    return T.full(shape, float("nan"), dtype=dtype, device="cuda:0")


def test_small_workload_gemm_bias_gelu():
    """64x256x256 GEMM + bias + GeLU, fp16, seed 0: the whole output."""
    T = torch()
    say("C1 64x256x256 gelu fp16", lf.plan_name(0, 64, 256, 256))
    d = synth.gemm_bias_gelu_small(seed=0)
    t = {k: dev_t(v, synth.F16) for k, v in d.items()}
    x = w64(d, synth.F16)
    want = oracle.gemm_epilogue(x["A"], x["W"], x["bias"], None, "gelu_tanh")
    got = to64(lf.gemm_epilogue(t["A"], t["W"], t["bias"], None, "gelu_tanh", out=nan_out((64, 256), T.float16)))
    assert_close(got, want, "C1")


def test_prefill_rmsnorm_linear_512x4096x4096():
    T = torch()
    say("C2 rmsnorm->linear 512x4096x4096 fp16", lf.plan_name(1, 512, 4096, 4096))
    d = synth.rmsnorm_linear(M=512, D=4096, N=4096, seed=0)
    t = {k: dev_t(v, synth.F16) for k, v in d.items()}
    x = w64(d, synth.F16)
    Y = to64(lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], EPS, out=nan_out((512, 4096), T.float16)))
    want = oracle.rmsnorm_gemm(x["X"], x["gamma"], EPS32, x["W"])
    assert_close(Y, want, "C2 whole output")


@pytest.mark.parametrize("M", [512, 1024, 2048, 4096])
def test_gemm_bias_gelu_sweep(M):
    T = torch()
    say("C3 gelu sweep M=%d" % M, lf.plan_name(0, M, 4096, 4096))
    d = synth.gemm_epilogue_sweep(M, seed=0)
    t = {k: dev_t(v, synth.F16) for k, v in d.items()}
    Y = to64(lf.gemm_epilogue(t["A"], t["W"], t["bias"], None, "gelu_tanh", out=nan_out((M, 4096), T.float16)))
    x = w64(d, synth.F16)
    want = oracle.gemm_epilogue(x["A"], x["W"], x["bias"], None, "gelu_tanh")
    assert_close(Y, want, "C3 M=%d whole output" % M)


@pytest.mark.parametrize("variant", ["silu", "relu", "residual"])
def test_gemm_epilogue_variants_4096(variant):
    T = torch()
    M = 4096
    say("C3 variant", variant, lf.plan_name(0, M, 4096, 4096))
    d = synth.gemm_epilogue_sweep(M, seed=0, residual=(variant == "residual"))
    t = {k: dev_t(v, synth.F16) for k, v in d.items()}
    x = w64(d, synth.F16)
    act = "none" if variant == "residual" else variant
    R = t.get("R")
    Y = to64(lf.gemm_epilogue(t["A"], t["W"], t["bias"], R, act, out=nan_out((M, 4096), T.float16)))
    want = oracle.gemm_epilogue(x["A"], x["W"], x["bias"], x["R"] if R is not None else None, act)
    assert_close(Y, want, "C3 %s whole output" % variant)


def swiglu_sensitivity(x):
    """|dH/dg| + |dH/du| for H = SiLU(g) u, at the oracle's gate and up projections
    g = RMSNorm(X) Wg and u = RMSNorm(X) Wu."""
    g = oracle.rmsnorm_gemm(x["X"], x["gamma"], EPS32, x["Wg"])
    u = oracle.rmsnorm_gemm(x["X"], x["gamma"], EPS32, x["Wu"])
    sig = 1.0 / (1.0 + np.exp(-g))
    return np.abs(u * sig * (1.0 + g * (1.0 - sig))) + np.abs(g * sig)


def test_swiglu_ffn_bf16_full():
    T = torch()
    M, D, F = 2048, 4096, 11008
    say("C4 swiglu ffn bf16", lf.plan_name(2, M, F, D, lf.BF16), lf.plan_name(0, M, D, F, lf.BF16))
    d = synth.swiglu_ffn(M=M, D=D, F=F, seed=0)
    t = {k: dev_t(v, synth.BF16) for k, v in d.items()}
    x = w64(d, synth.BF16)
    # kernel 1: H = SiLU(Xhat Wg) * (Xhat Wu)
    H16 = lf.rmsnorm_gemm_swiglu(t["X"], t["gamma"], t["Wg"], t["Wu"], EPS, out=nan_out((M, F), T.bfloat16))
    H32 = to64(lf.rmsnorm_gemm_swiglu(t["X"], t["gamma"], t["Wg"], t["Wu"], EPS, out_dtype=T.float32,
                                      out=nan_out((M, F), T.float32)))
    Hw = oracle.rmsnorm_swiglu(x["X"], x["gamma"], EPS32, x["Wg"], x["Wu"])
    # H = SiLU(g) * u is a nonlinear function of the two projections g and u,
    # which carry the tolerance: the bf16 rounding of the normalised operand
    # (which any bf16 matrix-core path has) perturbs g and u by about 1e-3,
    # and H moves by |dH/dg| |dg| + |dH/du| |du|.  So H's error is compared
    # after dividing by max(1, |dH/dg| + |dH/du|) at the oracle's g and u.
    # The block output Y below is held to the plain absolute tolerance.
    scale = np.maximum(1.0, swiglu_sensitivity(x))
    assert_close(H32 / scale, Hw / scale, "C4 k1 f32out (relative to H's sensitivity to g and u)")
    Hg = to64(H16)
    check_bf16_output(Hg, H32, Hw, "C4 k1")
    # kernel 2 on the H the GPU produced: Y = H Wd + b + X
    Y32 = to64(lf.gemm_epilogue(H16, t["Wd"], t["bias"], t["X"], "none", out_dtype=T.float32,
                                out=nan_out((M, D), T.float32)))
    want2 = oracle.gemm_epilogue(Hg, x["Wd"], x["bias"], x["X"], "none")
    assert_close(Y32, want2, "C4 k2 f32out")
    # whole block against the oracle's unrounded FFN: the oracle's down
    # projection applied to the oracle's H (the composition swiglu_ffn defines)
    want = oracle.gemm_epilogue(Hw, x["Wd"], x["bias"], x["X"], "none")
    assert_close(Y32, want, "C4 block f32out")
    Y16 = to64(lf.gemm_epilogue(H16, t["Wd"], t["bias"], t["X"], "none", out=nan_out((M, D), T.bfloat16)))
    check_bf16_output(Y16, Y32, want, "C4 block")


def test_swiglu_gate_up_fp16_full_plain_bound():
    """The C4 gate/up shape in fp16, whole output against the plain absolute
    bound: H reaches |H| ~ 20 here as in bf16, and with fp16's finer rounding
    of the normalised operand its error stays inside 1.5e-2 / 1.5e-3 without
    the sensitivity scaling the bf16 workload needs."""
    T = torch()
    M, D, F = 2048, 4096, 11008
    say("C4 gate/up fp16 full", lf.plan_name(2, M, F, D))
    d = synth.swiglu_ffn(M=M, D=D, F=F, seed=0, dtype=synth.F16)
    t = {k: dev_t(v, synth.F16) for k, v in d.items()}
    x = w64(d, synth.F16)
    H32 = to64(lf.rmsnorm_gemm_swiglu(t["X"], t["gamma"], t["Wg"], t["Wu"], EPS, out_dtype=T.float32,
                                      out=nan_out((M, F), T.float32)))
    Hw = oracle.rmsnorm_swiglu(x["X"], x["gamma"], EPS32, x["Wg"], x["Wu"])
    say("  max |H| %.2f" % float(np.abs(Hw).max()))
    assert float(np.abs(Hw).max()) > 8.0
    assert_close(H32, Hw, "C4 k1 fp16 f32out, plain bound")


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("D", [1024, 2048, 4096])
@pytest.mark.parametrize("B", [1, 32, 128, 512, 1024])
def test_decode_rmsnorm_linear_sweep(B, D, dtype):
    T = torch()
    say("C5 decode B=%d D=%d %s" % (B, D, dtype), lf.plan_name(1, B, D, D, dtype == synth.BF16))
    d = synth.decode_rmsnorm_linear(B, D, seed=0, dtype=dtype)
    t = {k: dev_t(v, dtype) for k, v in d.items()}
    x = w64(d, dtype)
    want = oracle.rmsnorm_gemm(x["X"], x["gamma"], EPS32, x["W"])
    if dtype == synth.F16:
        Y = to64(lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], EPS, out=nan_out((B, D), T.float16)))
        assert_close(Y, want, "C5 f16 whole output")
    else:
        Y = to64(lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], EPS, out_dtype=T.float32,
                                 out=nan_out((B, D), T.float32)))
        assert_close(Y, want, "C5 bf16 f32out whole output")
        Y16 = to64(lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], EPS, out=nan_out((B, D), T.bfloat16)))
        check_bf16_output(Y16, Y, want, "C5")


def test_largest_accepted_shape_whole_output():
    """M = 131064, K = N = 4096: M*K is just under the 2^29-element limit of the
    ABI (A and Y are 1 GiB each in fp16) and the last 256-row tile is ragged.
    A repeats a seeded 4096-row block, so the oracle's output for that block
    is the expected value of every row; all 131064 rows are compared (on the
    device, block by block), for the GEMM + bias + GeLU and for RMSNorm ->
    Linear."""
    T = torch()
    M, K, N, base_rows = 131064, 4096, 4096, 4096
    assert M * K < (1 << 29) and (M + 8) * K >= (1 << 29)
    say("largest shape", M, K, N, lf.plan_name(0, M, N, K), lf.plan_name(1, M, N, K))
    d = synth.rmsnorm_linear(M=base_rows, D=K, N=N, seed=27)
    b = synth.to_bits(synth.generator(28).standard_normal(N) * 0.1, synth.F16)
    Xb = dev_t(d["X"], synth.F16)
    X = Xb.repeat((M + base_rows - 1) // base_rows, 1)[:M].contiguous()
    W, g, bias = dev_t(d["W"], synth.F16), dev_t(d["gamma"], synth.F16), dev_t(b, synth.F16)
    x = w64(d, synth.F16)

    def compare(Y, want64, what):
        want = T.from_numpy(want64).to("cuda:0")
        mx, tot = 0.0, 0.0
        for r0 in range(0, M, base_rows):
            blk = Y[r0:r0 + base_rows]
            diff = (blk.double() - want[:blk.shape[0]]).abs()
            assert bool(T.isfinite(blk).all()), "%s: non-finite output in rows %d.." % (what, r0)
            mx = max(mx, float(diff.max()))
            tot += float(diff.sum())
        mean = tot / (M * N)
        say("  %s max_abs_err=%.3e mean_abs_err=%.3e" % (what, mx, mean))
        assert mx <= 1.5e-2 and mean <= 1.5e-3, (what, mx, mean)

    Y = lf.gemm_epilogue(X, W, bias, None, "gelu_tanh", out_dtype=T.float32, out=nan_out((M, N), T.float32))
    compare(Y, oracle.gemm_epilogue(x["X"], x["W"], synth.widen(b, synth.F16), None, "gelu_tanh"), "gelu all rows")
    del Y
    Y = lf.rmsnorm_gemm(X, g, W, EPS, out_dtype=T.float32, out=nan_out((M, N), T.float32))
    compare(Y, oracle.rmsnorm_gemm(x["X"], x["gamma"], EPS32, x["W"]), "rms all rows")
    del Y, X
