"""LayerNorm -> GEMM and the prologue-bias GEMM against the fp64 oracle (needs
an MI355X).

fuse_layernorm_gemm: Y = act(LayerNorm(X) W + bias), the layernorm_gemm
pattern of the "llm-fusion-compiler" pattern table.  fuse_gemm_prologue_bias:
Y = act((A + b) W + bias) + R, the deplodock post's Loop IR example
relu((x + bias) @ w).  Both run forced to each tile that carries them in turn
(the register-staged tiles; the 4 x 1 wave LDS-DMA tiles, with and without
split K, where K is a multiple of 64) over ragged shapes (including K not a
multiple of 64 for the register-staged tiles), every activation and both
dtypes, and at full size in the automatic plan; the whole output is compared,
written into NaN-filled buffers; integer data checks the plumbing of both
prologues bit for bit.  Tolerance:
max_abs_err <= 1.5e-2 and mean_abs_err <= 1.5e-3 (bf16 judged on a float32
output).  Rows with a mean far from zero check that LayerNorm centres before
it rounds; operands past the fp16 range check the tile's exact fallback.
"""
import numpy as np
import pytest

import gemm_epilogue_fuse_amd as lf
import oracle
import synth
from parity_util import assert_close, base, dev_t, fitk, say, to64

pytestmark = pytest.mark.gpu

EPS = 1e-5
EPS32 = float(np.float32(EPS))
ACTS = ["none", "relu", "gelu_tanh", "silu"]
PRO_PLANS = ["", "reg_256x256x64", "reg_128x128x64", "dma_256x256x32_s4", "dma_256x128x64_s3",
             "dma_256x128x64_s3:k2", "dma_128x128x64_s4", "dma_128x128x64_s4:k3", "dma_256x256x32_s4_w8",
             "dma_256x128x64_s3_w8", "dma_256x128x64_s3_w8:k2"]


@pytest.fixture(params=PRO_PLANS)
def pro_plan(request):
    lf.set_plan(request.param)
    yield request.param
    lf.set_plan(None)


def check_plan(plan, op, M, N, K):
    """The forced plan is the one that runs (K is fitted to it); a plan that
    does not carry this prologue skips the case."""
    if plan and not lf.lib().fuse_plan_applies(op, M, N, K, lf.F16, base(plan).encode()):
        pytest.skip("%s does not carry prologue op %d" % (plan, op))
    name = lf.plan_name(op, M, N, K)
    if plan:
        assert base(name) == base(plan), (plan, name)
    return name


def nan_out(shape, dtype):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda:0")


def ln_inputs(M, K, N, dtype, seed, mean_scale=0.0):
    """X rows N(mu_m, s_m) with per-row scale s_m in [0.5, 2] and mean mu_m =
    mean_scale * N(0,1) * s_m; gamma = 1 + N(0,0.1), beta ~ N(0,0.1), W ~
    N(0, 1/64) as in the GEMM + epilogue sweep (unit-scale outputs at K = 4096,
    smaller at smaller K), bias ~ N(0, 0.1).  (With W ~ N(0, 1/sqrt(K)) the
    outputs keep unit scale at every K, and the bf16 rounding of the
    normalised operand alone puts the mean error near 1.3e-3 for any bf16
    kernel: a handful of outputs then passes 1.5e-3 by chance.)"""
    g = synth.generator(seed)
    s = 0.5 + 1.5 * g.random((M, 1))
    X = (synth.normal(g, (M, K), 1.0) + mean_scale * synth.normal(g, (M, 1), 1.0)) * s
    gamma = synth.normal(g, (K,), 0.1, 1.0)
    beta = synth.normal(g, (K,), 0.1)
    W = synth.normal(g, (K, N), 1.0 / 64.0)
    b = synth.normal(g, (N,), 0.1)
    return {k: synth.to_bits(v, dtype) for k, v in (("X", X), ("gamma", gamma), ("beta", beta), ("W", W),
                                                     ("bias", b))}


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("M,N,K", [(300, 392, 328), (65, 136, 520), (1, 8, 64), (37, 72, 4672)])
def test_layernorm_gemm_ragged(pro_plan, dtype, act, M, N, K):
    import torch
    K = fitk(pro_plan, K)
    say("ln-gemm", pro_plan or "auto", check_plan(pro_plan, 3, M, N, K), dtype, act, M, N, K)
    d = ln_inputs(M, K, N, dtype, seed=81 + M, mean_scale=3.0)
    t = {k: dev_t(v, dtype) for k, v in d.items()}
    x = {k: synth.widen(v, dtype) for k, v in d.items()}
    for with_beta, with_bias in ((True, True), (False, False)):
        want = oracle.layernorm_gemm(x["X"], x["gamma"], EPS32, x["W"], x["beta"] if with_beta else None,
                                     x["bias"] if with_bias else None, act)
        args = (t["X"], t["gamma"], t["W"], EPS, t["beta"] if with_beta else None, t["bias"] if with_bias else None,
                act)
        got = to64(lf.layernorm_gemm(*args, out_dtype=torch.float32, out=nan_out((M, N), torch.float32)))
        assert_close(got, want, "f32out beta=%d bias=%d" % (with_beta, with_bias))
        if dtype == synth.F16:
            got16 = to64(lf.layernorm_gemm(*args, out=nan_out((M, N), torch.float16)))
            assert_close(got16, want, "f16out")


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_layernorm_gemm_offset_and_range(pro_plan, dtype):
    """Rows with a mean of 100 standard deviations, rows at 2^-10 and 2^8 scale,
    and one gamma of 30000 that pushes the normalised value past the fp16
    maximum (its W row is 1e-5, so outputs stay of unit scale): that tile
    falls back to the exact path."""
    import torch
    M, K, N = 520, 256, 136
    g = synth.generator(90)
    Z = synth.normal(g, (M, K), 1.0)
    scale = np.where(np.arange(M) % 3 == 0, 2.0 ** -10, np.where(np.arange(M) % 3 == 1, 1.0, 2.0 ** 8))[:, None]
    X = (Z + 100.0 * (np.arange(M) % 2 == 0)[:, None]) * scale
    gamma = synth.normal(g, (K,), 0.1, 1.0)
    beta = synth.normal(g, (K,), 0.1)
    W = synth.normal(g, (K, N), 1.0 / 64.0)
    if dtype == synth.F16:
        gamma[7] = 30000.0
        W[7] *= 1e-5
    bits = {k: synth.to_bits(v, dtype) for k, v in (("X", X), ("gamma", gamma), ("beta", beta), ("W", W))}
    t = {k: dev_t(v, dtype) for k, v in bits.items()}
    x = {k: synth.widen(v, dtype) for k, v in bits.items()}
    say("ln-gemm offset/range", dtype, check_plan(pro_plan, 3, M, N, K))
    want = oracle.layernorm_gemm(x["X"], x["gamma"], EPS32, x["W"], x["beta"], None, "gelu_tanh")
    got = to64(lf.layernorm_gemm(t["X"], t["gamma"], t["W"], EPS, t["beta"], None, "gelu_tanh",
                                 out_dtype=torch.float32, out=nan_out((M, N), torch.float32)))
    assert_close(got, want, "offset and range rows")


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_layernorm_gemm_rows_outside_the_window(pro_plan, dtype):
    """eps = 0 and rows whose variance lies outside the fast path's window
    (fp16: rows at 2^-14 scale, var + eps below 2^-24; bf16: rows at 2^60 and
    2^-70 scale, var outside [2^-120, 2^100]) between ordinary rows: their
    tiles take the exact path, the others the fast one."""
    import torch
    M, K, N = 300, 192, 136
    g = synth.generator(93)
    Z = synth.normal(g, (M, K), 1.0)
    odd = 2.0 ** -14 if dtype == synth.F16 else np.where(np.arange(M) % 2 == 0, 2.0 ** 60, 2.0 ** -70)[:, None]
    scale = np.where((np.arange(M) % 7 == 3)[:, None], odd, 1.0)
    X = (Z + 0.5) * scale
    gamma = synth.normal(g, (K,), 0.1, 1.0)
    beta = synth.normal(g, (K,), 0.1)
    W = synth.normal(g, (K, N), 1.0 / 64.0)
    bits = {k: synth.to_bits(v, dtype) for k, v in (("X", X), ("gamma", gamma), ("beta", beta), ("W", W))}
    t = {k: dev_t(v, dtype) for k, v in bits.items()}
    x = {k: synth.widen(v, dtype) for k, v in bits.items()}
    say("ln-gemm window rows", dtype, check_plan(pro_plan, 3, M, N, K))
    want = oracle.layernorm_gemm(x["X"], x["gamma"], 0.0, x["W"], x["beta"], None, "silu")
    got = to64(lf.layernorm_gemm(t["X"], t["gamma"], t["W"], 0.0, t["beta"], None, "silu",
                                 out_dtype=torch.float32, out=nan_out((M, N), torch.float32)))
    assert_close(got, want, "rows outside the window")


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_layernorm_gemm_full_size(dtype):
    """2048 x 4096 -> 4096, GeLU, the automatic plan, whole output."""
    import torch
    M, K, N = 2048, 4096, 4096
    say("ln-gemm full size", dtype, lf.plan_name(3, M, N, K))
    d = ln_inputs(M, K, N, dtype, seed=91)
    t = {k: dev_t(v, dtype) for k, v in d.items()}
    x = {k: synth.widen(v, dtype) for k, v in d.items()}
    want = oracle.layernorm_gemm(x["X"], x["gamma"], EPS32, x["W"], x["beta"], x["bias"], "gelu_tanh")
    got = to64(lf.layernorm_gemm(t["X"], t["gamma"], t["W"], EPS, t["beta"], t["bias"], "gelu_tanh",
                                 out_dtype=torch.float32, out=nan_out((M, N), torch.float32)))
    assert_close(got, want, "whole output f32out")


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("M,N,K", [(300, 392, 328), (65, 136, 520), (7, 24, 64)])
def test_layernorm_gemm_integer_plumbing_bit_exact(pro_plan, dtype, M, N, K):
    """eps = 0 and rows of +-1 or +-2 with exactly zero mean (var 1 or 4, so
    1/s = 1 or 1/2 exactly), small integer gamma, beta, W, bias: every
    operand, product and partial sum is exact, so the whole float32 output
    equals the oracle bit for bit on every tile (plumbing of the row records,
    the gamma/beta slots and the row factor)."""
    import torch
    K = fitk(pro_plan, K)
    K -= K % 2
    say("ln-gemm integer plumbing", dtype, check_plan(pro_plan, 3, M, N, K), M, N, K)
    g = synth.generator(M * 13 + K)
    X = np.tile(np.concatenate([np.ones(K // 2), -np.ones(K // 2)]), (M, 1))
    X = np.array([g.permutation(r) for r in X]) * np.where(np.arange(M) % 2 == 0, 1.0, 2.0)[:, None]
    gamma = g.integers(-2, 3, K).astype(np.float64)
    beta = g.integers(-2, 3, K).astype(np.float64)
    W = g.integers(-1, 2, (K, N)).astype(np.float64)
    b = g.integers(-50, 51, N).astype(np.float64)
    bits = {k: synth.to_bits(v, dtype) for k, v in (("X", X), ("gamma", gamma), ("beta", beta), ("W", W), ("b", b))}
    t = {k: dev_t(v, dtype) for k, v in bits.items()}
    for act in ("none", "relu"):
        want = oracle.layernorm_gemm(X, gamma, 0.0, W, beta, b, act)
        got = to64(lf.layernorm_gemm(t["X"], t["gamma"], t["W"], 0.0, t["beta"], t["b"], act,
                                     out_dtype=torch.float32, out=nan_out((M, N), torch.float32)))
        assert np.array_equal(got, want), (act, np.abs(got - want).max())


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("M,N,K", [(300, 392, 328), (65, 136, 520), (7, 24, 64)])
def test_prologue_bias_integer_plumbing_bit_exact(pro_plan, dtype, M, N, K):
    """Small integer A, input bias, W, bias and residual: x + b and every
    partial sum are exact, so the whole float32 output equals the oracle bit
    for bit on every tile (plumbing of the bias slot against the A chunks)."""
    import torch
    K = fitk(pro_plan, K)
    say("prologue-bias integer plumbing", dtype, check_plan(pro_plan, 4, M, N, K), M, N, K)
    g = synth.generator(M * 17 + K)
    A = g.integers(-2, 3, (M, K)).astype(np.float64)
    ab = g.integers(-2, 3, K).astype(np.float64)
    W = g.integers(-1, 2, (K, N)).astype(np.float64)
    b = g.integers(-50, 51, N).astype(np.float64)
    R = g.integers(-50, 51, (M, N)).astype(np.float64)
    bits = {k: synth.to_bits(v, dtype) for k, v in (("A", A), ("ab", ab), ("W", W), ("b", b), ("R", R))}
    t = {k: dev_t(v, dtype) for k, v in bits.items()}
    for act in ("none", "relu"):
        want = oracle.prologue_bias_gemm(A, ab, W, b, R, act)
        got = to64(lf.gemm_prologue_bias(t["A"], t["ab"], t["W"], t["b"], t["R"], act, out_dtype=torch.float32,
                                         out=nan_out((M, N), torch.float32)))
        assert np.array_equal(got, want), (act, np.abs(got - want).max())


def pb_inputs(M, K, N, dtype, seed):
    """A ~ N(0,1) and abias ~ N(0,1) (the page's example draws both from randn),
    W ~ N(0, 1/64) as in the GEMM + epilogue sweep, bias ~ N(0,0.1), R ~ N(0,1).
    (x + b has standard deviation sqrt(2); with W ~ N(0, 1/sqrt(K)) the output
    would have unit scale and the bf16 rounding of the operand alone would put
    the mean error at the 1.5e-3 bound for any bf16 kernel.)"""
    g = synth.generator(seed)
    fields = (("A", synth.normal(g, (M, K), 1.0)), ("abias", synth.normal(g, (K,), 1.0)),
              ("W", synth.normal(g, (K, N), 1.0 / 64.0)), ("bias", synth.normal(g, (N,), 0.1)),
              ("R", synth.normal(g, (M, N), 1.0)))
    return {k: synth.to_bits(v, dtype) for k, v in fields}


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("M,N,K", [(300, 392, 328), (65, 136, 520), (16, 16, 64)])
def test_prologue_bias_ragged(pro_plan, dtype, act, M, N, K):
    import torch
    K = fitk(pro_plan, K)
    say("prologue-bias", pro_plan or "auto", check_plan(pro_plan, 4, M, N, K), dtype, act, M, N, K)
    d = pb_inputs(M, K, N, dtype, seed=95 + K)
    t = {k: dev_t(v, dtype) for k, v in d.items()}
    x = {k: synth.widen(v, dtype) for k, v in d.items()}
    for bias, res in ((True, True), (False, False), (True, False)):
        want = oracle.prologue_bias_gemm(x["A"], x["abias"], x["W"], x["bias"] if bias else None,
                                         x["R"] if res else None, act)
        args = (t["A"], t["abias"], t["W"], t["bias"] if bias else None, t["R"] if res else None, act)
        got = to64(lf.gemm_prologue_bias(*args, out_dtype=torch.float32, out=nan_out((M, N), torch.float32)))
        assert_close(got, want, "f32out bias=%d res=%d" % (bias, res))
        if dtype == synth.F16:
            got16 = to64(lf.gemm_prologue_bias(*args, out=nan_out((M, N), torch.float16)))
            assert_close(got16, want, "f16out bias=%d res=%d" % (bias, res))


def test_prologue_bias_worked_example_and_overflow(pro_plan):
    """The page's relu((x + bias) @ w) at (16, 64) x (64, 16), then a call whose
    x + b passes the fp16 maximum in a few elements (60000 + 8000; their W rows
    are 1e-5): the affected tile takes the exact path."""
    import torch
    dt = synth.F16
    g = synth.generator(97)
    x, ab, w = synth.normal(g, (16, 64), 1.0), synth.normal(g, (64,), 1.0), synth.normal(g, (64, 16), 0.125)
    bits = {k: synth.to_bits(v, dt) for k, v in (("x", x), ("ab", ab), ("w", w))}
    t = {k: dev_t(v, dt) for k, v in bits.items()}
    xv = {k: synth.widen(v, dt) for k, v in bits.items()}
    say("prologue-bias worked example", lf.plan_name(4, 16, 16, 64))
    got = to64(lf.gemm_prologue_bias(t["x"], t["ab"], t["w"], act="relu", out=nan_out((16, 16), torch.float16)))
    assert_close(got, oracle.prologue_bias_gemm(xv["x"], xv["ab"], xv["w"], act_kind="relu"), "worked example")
    M, K, N = 300, 192, 136
    say("  overflow case", check_plan(pro_plan, 4, M, N, K))
    A = synth.normal(g, (M, K), 1.0)
    abias = synth.normal(g, (K,), 1.0)
    W = synth.normal(g, (K, N), 1.0 / np.sqrt(K))
    A[5, 3] = 60000.0
    abias[3] = 8000.0
    W[3] *= 1e-5
    bits = {k: synth.to_bits(v, dt) for k, v in (("A", A), ("ab", abias), ("W", W))}
    t = {k: dev_t(v, dt) for k, v in bits.items()}
    xv = {k: synth.widen(v, dt) for k, v in bits.items()}
    want = oracle.prologue_bias_gemm(xv["A"], xv["ab"], xv["W"], act_kind="silu")
    got = to64(lf.gemm_prologue_bias(t["A"], t["ab"], t["W"], act="silu", out_dtype=torch.float32,
                                     out=nan_out((M, N), torch.float32)))
    assert_close(got, want, "x + b past the fp16 maximum")


def test_prologue_bias_bf16_overflow(pro_plan):
    """bf16: a few x + b past the bf16 maximum but inside float32's (2.5e38 +
    9e37; their W row is scaled by 1e-38): the rounded operand is infinite, so
    the affected tiles take the exact path (float32 operand)."""
    import torch
    dt = synth.BF16
    g = synth.generator(98)
    M, K, N = 300, 192, 136
    A = synth.normal(g, (M, K), 1.0)
    abias = synth.normal(g, (K,), 1.0)
    W = synth.normal(g, (K, N), 1.0 / 64.0)
    A[5, 3] = 2.5e38
    A[250, 3] = 2.5e38
    abias[3] = 9e37
    W[3] *= 1e-38
    bits = {k: synth.to_bits(v, dt) for k, v in (("A", A), ("ab", abias), ("W", W))}
    t = {k: dev_t(v, dt) for k, v in bits.items()}
    xv = {k: synth.widen(v, dt) for k, v in bits.items()}
    say("prologue-bias bf16 overflow", check_plan(pro_plan, 4, M, N, K))
    want = oracle.prologue_bias_gemm(xv["A"], xv["ab"], xv["W"], act_kind="gelu_tanh")
    got = to64(lf.gemm_prologue_bias(t["A"], t["ab"], t["W"], act="gelu_tanh", out_dtype=torch.float32,
                                     out=nan_out((M, N), torch.float32)))
    assert_close(got, want, "x + b past the bf16 maximum")


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_prologue_bias_full_size(dtype):
    """4096^3 GEMM + bias + GeLU with an input bias, the automatic plan, whole
    output (fp16 output for fp16, float32 output for bf16)."""
    import torch
    M = N = K = 4096
    code = lf.BF16 if dtype == synth.BF16 else lf.F16
    say("prologue-bias full size", dtype, lf.plan_name(4, M, N, K, code))
    d = pb_inputs(M, K, N, dtype, seed=99)
    t = {k: dev_t(v, dtype) for k, v in d.items()}
    x = {k: synth.widen(v, dtype) for k, v in d.items()}
    want = oracle.prologue_bias_gemm(x["A"], x["abias"], x["W"], x["bias"], None, "gelu_tanh")
    if dtype == synth.F16:
        got = to64(lf.gemm_prologue_bias(t["A"], t["abias"], t["W"], t["bias"], None, "gelu_tanh",
                                         out=nan_out((M, N), torch.float16)))
    else:
        got = to64(lf.gemm_prologue_bias(t["A"], t["abias"], t["W"], t["bias"], None, "gelu_tanh",
                                         out_dtype=torch.float32, out=nan_out((M, N), torch.float32)))
    assert_close(got, want, "whole output")
