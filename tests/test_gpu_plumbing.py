"""Bit-exact shape and index plumbing of the HIP path (needs an MI355X).

Inputs are chosen so that every fp32 partial sum is exact in any order
(identity and permutation weights, small integers, power-of-two RMS rows),
so the GPU must equal the oracle bit for bit: a wrong tile index, a dropped
M/N/K tail, a transposed operand or a wrong accumulator-to-row mapping shows
up as a mismatch.  Each tile plan is forced in turn so that every kernel
configuration crosses tile edges and ragged tails at small sizes.
"""
import numpy as np
import pytest

import gemm_epilogue_fuse_amd as lf
import oracle
import synth
from parity_util import DUAL_PLANS, PLANS, base, dev_t, fitk, say, to64

pytestmark = pytest.mark.gpu

DTYPES = [synth.F16, synth.BF16]
ONE = {synth.F16: 0x3C00, synth.BF16: 0x3F80}
SHAPES = [(1, 8, 8), (7, 24, 40), (65, 136, 72), (129, 264, 200), (300, 392, 328), (520, 776, 264)]


@pytest.fixture(params=PLANS)
def plan(request):
    lf.set_plan(request.param)
    yield request.param
    lf.set_plan(None)


def eye_bits(K, N, dtype):
    b = np.zeros((K, N), dtype=np.uint16)
    idx = np.arange(min(K, N))
    b[idx, idx] = ONE[dtype]
    return b


def rand_bits(shape, dtype, seed):
    return synth.to_bits(synth.generator(seed).standard_normal(shape), dtype)


def nan_filled(shape, dtype):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda:0")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,K", [(1, 8), (7, 40), (65, 136), (300, 328), (513, 264)])
def test_identity_weight_returns_input(plan, dtype, M, K):
    K = fitk(plan, K)
    assert base(lf.plan_name(0, M, K, K)) == base(plan)
    say("identity", plan, dtype, M, K)
    A = rand_bits((M, K), dtype, 100 + M)
    At = dev_t(A, dtype)
    I = dev_t(eye_bits(K, K, dtype), dtype)
    Y = lf.gemm_epilogue(At, I, out=nan_filled((M, K), At.dtype))
    assert np.array_equal(to64(Y), synth.widen(A, dtype))
    Y = lf.gemm_epilogue(At, I, act="relu")
    assert np.array_equal(to64(Y), np.maximum(synth.widen(A, dtype), 0.0))


@pytest.mark.parametrize("dtype", DTYPES)
def test_permutation_weights(plan, dtype):
    g = synth.generator(5)
    for M, K in ((33, 24), (260, 136)):
        K = fitk(plan, K)
        say("perm-cols", plan, dtype, M, K)
        A = rand_bits((M, K), dtype, 200 + M)
        p = g.permutation(K)
        P = np.zeros((K, K), dtype=np.uint16)
        P[p, np.arange(K)] = ONE[dtype]
        Y = lf.gemm_epilogue(dev_t(A, dtype), dev_t(P, dtype))
        assert np.array_equal(to64(Y), synth.widen(A, dtype)[:, p])
    for M, N in ((24, 40), (264, 392)):
        M = fitk(plan, M)  # here M is also the reduction length
        say("perm-rows", plan, dtype, M, N)
        q = g.permutation(M)
        Q = np.zeros((M, M), dtype=np.uint16)
        Q[np.arange(M), q] = ONE[dtype]
        B = rand_bits((M, N), dtype, 300 + M)
        Y = lf.gemm_epilogue(dev_t(Q, dtype), dev_t(B, dtype))
        assert np.array_equal(to64(Y), synth.widen(B, dtype)[q])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_integer_data_bit_exact(plan, dtype, M, N, K):
    import torch
    K = fitk(plan, K)
    assert lf.plan_name(0, M, N, K) == plan
    say("integer", plan, dtype, M, N, K)
    g = synth.generator(M * 31 + N * 7 + K)
    A = g.integers(-1, 2, (M, K)).astype(np.float64)
    W = g.integers(-1, 2, (K, N)).astype(np.float64)
    b = g.integers(-100, 101, N).astype(np.float64)
    R = g.integers(-100, 101, (M, N)).astype(np.float64)
    bits = {k: synth.to_bits(v, dtype) for k, v in (("A", A), ("W", W), ("b", b), ("R", R))}
    t = {k: dev_t(v, dtype) for k, v in bits.items()}
    for act in ("none", "relu"):
        want = oracle.gemm_epilogue(A, W, b, R, act)
        # bf16 holds integers exactly only up to 256: check it with a float32 output
        out_dtype = torch.float32 if dtype == synth.BF16 else None
        Y = lf.gemm_epilogue(t["A"], t["W"], t["b"], t["R"], act, out_dtype=out_dtype,
                             out=nan_filled((M, N), out_dtype or t["A"].dtype))
        assert np.array_equal(to64(Y), want), (act, np.abs(to64(Y) - want).max())
        Y = lf.gemm_epilogue(t["A"], t["W"], None, None, act, out_dtype=torch.float32)
        assert np.array_equal(to64(Y), oracle.gemm_epilogue(A, W, None, None, act))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N,K", [(7, 24, 64), (129, 264, 200), (300, 136, 520)])
def test_rmsnorm_exact_rows(plan, dtype, M, N, K):
    # eps = 0 and rows of +-1 (mean square 1) or +-2 (mean square 4): r = 1 or
    # 1/2 exactly; with W = I the output is sign * gamma bit for bit.
    K = fitk(plan, K)
    assert lf.plan_name(1, M, N, K) == plan
    say("rms-exact", plan, dtype, M, N, K)
    g = synth.generator(9 + M)
    sign = g.choice([-1.0, 1.0], size=(M, K))
    scale = np.where(np.arange(M) % 2 == 0, 1.0, 2.0)[:, None]
    X = sign * scale
    gamma = synth.widen(synth.to_bits(1.0 + 0.1 * g.standard_normal(K), dtype), dtype)
    Wt = dev_t(eye_bits(K, N, dtype), dtype)
    Xt = dev_t(synth.to_bits(X, dtype), dtype)
    gt = dev_t(synth.to_bits(gamma, dtype), dtype)
    Y = lf.rmsnorm_gemm(Xt, gt, Wt, eps=0.0, out=nan_filled((M, N), Xt.dtype))
    want = (sign * gamma[None, :])[:, :N] if N <= K else np.pad(sign * gamma[None, :], ((0, 0), (0, N - K)))
    assert np.array_equal(to64(Y), want)
    # Scaling X by 2 changes nothing (power-of-two scaling is exact end to end)
    X2 = dev_t(synth.to_bits(2.0 * X, dtype), dtype)
    Y2 = lf.rmsnorm_gemm(X2, gt, Wt, eps=0.0)
    assert np.array_equal(to64(Y2), to64(Y))


@pytest.mark.parametrize("dtype", DTYPES)
def test_rmsnorm_scale_invariance_random(plan, dtype):
    say("rms-scale", plan, dtype)
    d = synth.rmsnorm_linear(M=130, D=fitk(plan, 264), N=136, seed=3, dtype=dtype)
    X = synth.widen(d["X"], dtype)
    # keep x*gamma out of the fp16 subnormal range, where rounding is absolute
    # rather than relative and doubling would not commute with it
    X = np.where(np.abs(X) < 1e-2, np.copysign(1e-2, X), X)
    d["X"] = synth.to_bits(X, dtype)
    t = {k: dev_t(v, dtype) for k, v in d.items()}
    Y1 = lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], eps=0.0, act="gelu_tanh")
    Y2 = lf.rmsnorm_gemm(dev_t(synth.to_bits(2.0 * X, dtype), dtype), t["gamma"], t["W"], eps=0.0,
                         act="gelu_tanh")
    assert np.array_equal(to64(Y1), to64(Y2))


@pytest.mark.parametrize("dtype", DTYPES)
def test_rmsnorm_unit_rms(plan, dtype):
    import torch
    say("rms-unit", plan, dtype)
    M, K = 96, 512
    assert lf.plan_name(1, M, K, K) == plan
    X = synth.to_bits(synth.generator(4).standard_normal((M, K)), dtype)
    ones = np.full(K, ONE[dtype], dtype=np.uint16)
    Y = lf.rmsnorm_gemm(dev_t(X, dtype), dev_t(ones, dtype), dev_t(eye_bits(K, K, dtype), dtype), eps=1e-6,
                        out_dtype=torch.float32)
    Xw = synth.widen(X, dtype)
    ms = np.mean(Xw * Xw, axis=1)
    rms_out = np.sqrt(np.mean(to64(Y) ** 2, axis=1))
    # the operand x*gamma is rounded to the input type before the product
    tol = 2e-3 if dtype == synth.F16 else 8e-3
    assert np.max(np.abs(rms_out - np.sqrt(ms / (ms + 1e-6)))) < tol


@pytest.fixture(params=DUAL_PLANS)
def dual_plan(request):
    lf.set_plan(request.param)
    yield request.param
    lf.set_plan(None)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K", [264, 320])
def test_swiglu_plumbing(dual_plan, dtype, K):
    import torch
    # Wg = Wu = I, gamma = 1, rows +-1, eps = 0: H = silu(x) * x exactly per element
    # (K = 264 runs the register-staged plan, K = 320 the DMA plan)
    say("swiglu-plumbing", dtype, K, lf.plan_name(2, 70, K, K))
    M = 70
    g = synth.generator(11)
    X = g.choice([-1.0, 1.0], size=(M, K))
    I = dev_t(eye_bits(K, K, dtype), dtype)
    ones = dev_t(np.full(K, ONE[dtype], dtype=np.uint16), dtype)
    H = lf.rmsnorm_gemm_swiglu(dev_t(synth.to_bits(X, dtype), dtype), ones, I, I, eps=0.0,
                               out_dtype=torch.float32)
    want = oracle.act(X, "silu") * X
    assert np.max(np.abs(to64(H) - want)) < 1e-6


def test_in_place_residual():
    say("in-place residual")
    d = synth.gemm_epilogue_sweep(M=200, N=264, K=136, residual=True)
    t = {k: dev_t(v, synth.F16) for k, v in d.items()}
    want = lf.gemm_epilogue(t["A"], t["W"], t["bias"], t["R"], "silu")
    R = t["R"].clone()
    got = lf.gemm_epilogue(t["A"], t["W"], t["bias"], R, "silu", out=R)
    assert got.data_ptr() == R.data_ptr()
    assert np.array_equal(to64(got), to64(want))


def test_zero_rows_noop():
    import torch
    A = torch.zeros((0, 64), dtype=torch.float16, device="cuda:0")
    W = torch.zeros((64, 64), dtype=torch.float16, device="cuda:0")
    Y = lf.gemm_epilogue(A, W)
    assert Y.shape == (0, 64)


@pytest.mark.parametrize("plan_name", PLANS)
@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_deterministic(plan_name, dtype):
    """Repeated calls on the same inputs agree bit for bit (split-K sums run in
    a fixed order; no fragment may be consumed before its LDS read lands)."""
    import torch
    lf.set_plan(plan_name)
    try:
        say("determinism", plan_name, dtype)
        d = synth.rmsnorm_linear(M=300, D=fitk(plan_name, 520), N=392, seed=1, dtype=dtype)
        t = {k: dev_t(v, dtype) for k, v in d.items()}
        ref = lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], act="gelu_tanh", out_dtype=torch.float32).clone()
        refg = lf.gemm_epilogue(t["X"], t["W"], act="relu", out_dtype=torch.float32).clone()
        for _ in range(20):
            y = lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], act="gelu_tanh", out_dtype=torch.float32)
            assert torch.equal(y.view(torch.int32), ref.view(torch.int32))
            y = lf.gemm_epilogue(t["X"], t["W"], act="relu", out_dtype=torch.float32)
            assert torch.equal(y.view(torch.int32), refg.view(torch.int32))
        assert bool(torch.isfinite(ref).all()) and bool(torch.isfinite(refg).all())
    finally:
        lf.set_plan(None)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_deterministic_swiglu(dual_plan, dtype):
    """The gate/up kernel scales A one sub-step ahead with hand-scheduled bf16
    code; repeated calls agree bit for bit (no value read before it lands)."""
    import torch
    M, F, K = 300, 392, 544
    say("determinism swiglu", dtype, lf.plan_name(2, M, F, K, lf.BF16 if dtype == "bf16" else lf.F16))
    d = synth.swiglu_ffn(M=M, D=K, F=F, seed=3, dtype=dtype)
    t = {k: dev_t(v, dtype) for k, v in d.items() if k in ("X", "gamma", "Wg", "Wu")}
    ref = lf.rmsnorm_gemm_swiglu(t["X"], t["gamma"], t["Wg"], t["Wu"], 1e-6, out_dtype=torch.float32).clone()
    for _ in range(20):
        y = lf.rmsnorm_gemm_swiglu(t["X"], t["gamma"], t["Wg"], t["Wu"], 1e-6, out_dtype=torch.float32)
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32))
    assert bool(torch.isfinite(ref).all())


@pytest.mark.parametrize("plan_name", ["dma_128x128x64_s4_g2:k2", "dma_64x128x64_s4_g2:k3", "dec_32x64:k3",
                                       "dma_256x128x64_s3_w8:k2", "wstrip_16x16", "auto-decode"])
def test_graph_replay_matches_eager(plan_name):
    """Calls captured in a HIP graph (on a stream that made one eager call
    first, so its split-K workspace exists) and replayed several times, with
    eager work between the replays, give the eager result bit for bit: the
    split-K arrival counters are back at zero after every call."""
    import torch
    auto = plan_name == "auto-decode"
    lf.set_plan(None if auto else plan_name)
    try:
        M, D, N = (1, 4096, 4096) if auto else (100, fitk(plan_name, 520), 392)
        if not auto:
            assert lf.plan_name(1, M, N, D) == plan_name
        say("graph replay", plan_name, M, D, N, lf.plan_name(1, M, N, D))
        d = synth.rmsnorm_linear(M=M, D=D, N=N, seed=4, dtype=synth.F16)
        t = {k: dev_t(v, synth.F16) for k, v in d.items()}
        ref = lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], act="silu", out_dtype=torch.float32).clone()
        outs = [torch.empty((M, N), dtype=torch.float32, device="cuda:0") for _ in range(2)]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], act="silu", out=outs[0], out_dtype=torch.float32)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for o in outs:
                lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], act="silu", out=o, out_dtype=torch.float32)
        for _ in range(4):
            for o in outs:
                o.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for o in outs:
                assert torch.equal(o.view(torch.int32), ref.view(torch.int32))
    finally:
        lf.set_plan(None)


# --------------------------------------------------------------------------- full sizes, automatic plans
#
# The multi-group tile order, uneven XCD remainders, split-K counts above 3
# and the decode kernel's long chunk lists only occur at full size.  Small
# integer data keeps every fp32 partial sum exact in any order, so the whole
# output must equal the oracle bit for bit (float32 output: the sums reach
# several thousand).

FULL_SHAPES = [(4096, 4096, 4096), (512, 4096, 4096), (2048, 4096, 11008), (2048, 11008, 4096),
               (1024, 4096, 4096), (128, 4096, 4096), (32, 4096, 4096), (1, 4096, 4096), (130, 4104, 2048)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N,K", FULL_SHAPES)
def test_integer_data_bit_exact_full_size(dtype, M, N, K):
    import torch
    say("integer full size", dtype, M, N, K, lf.plan_name(0, M, N, K, lf.BF16 if dtype == synth.BF16 else lf.F16))
    g = synth.generator(M + 3 * N + 7 * K)
    A = g.integers(-1, 2, (M, K)).astype(np.float64)
    W = g.integers(-1, 2, (K, N)).astype(np.float64)
    b = g.integers(-100, 101, N).astype(np.float64)
    R = g.integers(-100, 101, (M, N)).astype(np.float64)
    bits = {k: synth.to_bits(v, dtype) for k, v in (("A", A), ("W", W), ("b", b), ("R", R))}
    t = {k: dev_t(v, dtype) for k, v in bits.items()}
    want = oracle.gemm_epilogue(A, W, b, R, "relu")
    Y = lf.gemm_epilogue(t["A"], t["W"], t["b"], t["R"], "relu", out_dtype=torch.float32,
                         out=nan_filled((M, N), torch.float32))
    got = to64(Y)
    assert np.array_equal(got, want), np.nanmax(np.abs(got - want))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,K", [(512, 4096), (2048, 4096), (1, 4096), (32, 4096), (128, 2048), (1024, 1024)])
def test_rmsnorm_exact_rows_full_size(dtype, M, K):
    """eps = 0, rows of +-1 and +-2 (r = 1 and 1/2 exactly), W = I: the output
    is sign * gamma bit for bit, through the automatic plan (split K, decode
    chunks) at full size."""
    say("rms-exact full size", dtype, M, K, lf.plan_name(1, M, K, K, lf.BF16 if dtype == synth.BF16 else lf.F16))
    g = synth.generator(11 + M + K)
    sign = g.choice([-1.0, 1.0], size=(M, K))
    X = sign * np.where(np.arange(M) % 2 == 0, 1.0, 2.0)[:, None]
    gamma = synth.widen(synth.to_bits(1.0 + 0.1 * g.standard_normal(K), dtype), dtype)
    Xt = dev_t(synth.to_bits(X, dtype), dtype)
    Y = lf.rmsnorm_gemm(Xt, dev_t(synth.to_bits(gamma, dtype), dtype), dev_t(eye_bits(K, K, dtype), dtype),
                        eps=0.0, out=nan_filled((M, K), Xt.dtype))
    assert np.array_equal(to64(Y), sign * gamma[None, :])
