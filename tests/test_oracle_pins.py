"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test names the part of the oracle it pins and what pins it: the pages'
printed figures (``tests/golden``), closed forms, special inputs whose exact
result is known (identity, permutation, small integers), library routines
(numpy matmul, torch rms_norm, scipy erf / expit), and a pure-Python brute
force on tiny shapes.  None of these runs on a GPU.
"""
import math
import os

import numpy as np
import pytest
import scipy.special as sp
import torch

import oracle
from oracle import brute
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS32 = float(np.float32(1e-6))  # eps as the 32-bit value the library receives


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(None, 1)
            vals[k] = v
    return vals


# --------------------------------------------------------------------------
# Activations (pinned against the page's GeLU figure, erf/expit, closed forms)
# --------------------------------------------------------------------------

def test_gelu_tanh_deviation_matches_page_figure():
    g = _golden("gelu_tanh_deviation.txt")
    z = np.linspace(-8.0, 8.0, 320001)
    exact = 0.5 * z * (1.0 + sp.erf(z / math.sqrt(2.0)))
    dev = np.max(np.abs(oracle.act(z, "gelu_tanh") - exact))
    assert round(dev, int(g["decimals"])) == float(g["max_abs_deviation"])
    assert dev <= 5e-4  # tolerance against erf-GeLU stated for the operator


def test_gelu_tanh_closed_form_point():
    # Pick z where sqrt(2/pi)(z + 0.044715 z^3) = atanh(0.6); there tanh = 0.6,
    # so gelu(z) = 0.5 z (1 + 0.6) = 0.8 z.  The cubic is solved by numpy.roots.
    c = math.sqrt(2.0 / math.pi)
    target = math.atanh(0.6)
    roots = np.roots([0.044715 * c, 0.0, c, -target])
    z = float(roots[np.argmin(np.abs(roots.imag))].real)
    assert abs(oracle.act(np.array([z]), "gelu_tanh")[0] - 0.8 * z) < 1e-14


def test_gelu_odd_part_and_limits():
    z = np.linspace(-5, 5, 1001)
    g = oracle.act(z, "gelu_tanh")
    gm = oracle.act(-z, "gelu_tanh")
    # gelu(z) - gelu(-z) = z for any odd "tanh" inside: exact identity
    assert np.max(np.abs((g - gm) - z)) < 1e-13
    big = oracle.act(np.array([0.0, 12.0, -12.0]), "gelu_tanh")
    assert big[0] == 0.0 and abs(big[1] - 12.0) < 1e-12 and abs(big[2]) < 1e-12


def test_silu_against_expit_and_closed_forms():
    z = np.linspace(-30, 30, 6001)
    s = oracle.act(z, "silu")
    assert np.max(np.abs(s - z * sp.expit(z))) < 1e-13
    # sigma(ln 3) = 3/4  =>  silu(ln 3) = 0.75 ln 3
    assert abs(oracle.act(np.array([math.log(3.0)]), "silu")[0] - 0.75 * math.log(3.0)) < 1e-15
    # silu(z) - silu(-z) = z
    assert np.max(np.abs(s - oracle.act(-z, "silu") - z)) < 1e-12
    assert oracle.act(np.array([0.0]), "silu")[0] == 0.0


def test_relu_and_none():
    z = np.array([-3.0, -0.0, 0.0, 1e-300, 2.5])
    assert np.array_equal(oracle.act(z, "relu"), np.array([0.0, 0.0, 0.0, 1e-300, 2.5]))
    assert np.array_equal(oracle.act(z, "none"), z)


def test_act_codes_match_public_enumeration():
    # The public header fixes NONE=0, RELU=1, GELU_TANH=2, SILU=3; the oracle's
    # own codes must agree so that tests can pass one integer to both.
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "fuse.h")).read()
    for name, code in (("NONE", 0), ("RELU", 1), ("GELU_TANH", 2), ("SILU", 3)):
        assert "FUSE_ACT_%s = %d" % (name, code) in hdr
        assert oracle.ACT_CODES[name.lower()] == code


# --------------------------------------------------------------------------
# GEMM + epilogue
# --------------------------------------------------------------------------

def test_identity_weight_returns_input():
    g = synth.generator(1)
    for M, K in ((1, 8), (7, 16), (65, 64)):
        A = g.standard_normal((M, K))
        I = np.eye(K)
        assert np.array_equal(oracle.gemm_epilogue(A, I), A)
        assert np.array_equal(oracle.gemm_epilogue(A, I, act_kind="relu"), np.maximum(A, 0.0))


def test_permutation_weights_permute():
    g = synth.generator(2)
    M, K = 33, 24
    A = g.standard_normal((M, K))
    p = g.permutation(K)
    P = np.zeros((K, K))
    P[p, np.arange(K)] = 1.0  # column j of A @ P is column p[j] of A
    assert np.array_equal(oracle.gemm_epilogue(A, P), A[:, p])
    q = g.permutation(M)
    Q = np.zeros((M, M))
    Q[np.arange(M), q] = 1.0  # row i of Q @ B is row q[i] of B
    B = g.standard_normal((M, 16))
    assert np.array_equal(oracle.gemm_epilogue(Q, B), B[q])


@pytest.mark.parametrize("shape", [(1, 8, 8), (17, 40, 24), (64, 256, 136)])
def test_integer_data_is_exact(shape):
    M, K, N = shape
    g = synth.generator(3)
    A = g.integers(-1, 2, (M, K))
    W = g.integers(-1, 2, (K, N))
    b = g.integers(-50, 51, (N,))
    R = g.integers(-50, 51, (M, N))
    want = A.astype(np.int64) @ W.astype(np.int64) + b
    got = oracle.gemm_epilogue(A, W, b, R, "none")
    assert np.array_equal(got, (want + R).astype(np.float64))
    got_relu = oracle.gemm_epilogue(A, W, b, R, "relu")
    assert np.array_equal(got_relu, (np.maximum(want, 0) + R).astype(np.float64))


def test_gemm_matches_numpy_matmul():
    g = synth.generator(4)
    A = g.standard_normal((37, 96))
    W = g.standard_normal((96, 72))
    b = g.standard_normal(72)
    R = g.standard_normal((37, 72))
    ref = A @ W
    got = oracle.gemm_epilogue(A, W)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    # bias before activation, residual after: check against composed library calls
    got2 = oracle.gemm_epilogue(A, W, b, R, "silu")
    z = ref + b
    assert np.max(np.abs(got2 - (z * sp.expit(z) + R))) < 1e-11


def test_bias_enters_before_activation():
    # With A = 0, Y = act(bias) + R: a bias added after the activation would
    # give relu(0) + bias = bias instead.
    N = 16
    b = np.linspace(-2, 2, N)
    Y = oracle.gemm_epilogue(np.zeros((3, 8)), np.ones((8, N)), b, None, "relu")
    assert np.array_equal(Y, np.tile(np.maximum(b, 0), (3, 1)))


# --------------------------------------------------------------------------
# RMSNorm prologue
# --------------------------------------------------------------------------

def test_rmsnorm_gamma1_has_unit_rms():
    g = synth.generator(5)
    X = g.standard_normal((64, 512))
    Y = oracle.rmsnorm_gemm(X, np.ones(512), EPS32, np.eye(512))
    ms = np.mean(X * X, axis=1)
    rms_out = np.sqrt(np.mean(Y * Y, axis=1))
    assert np.max(np.abs(rms_out - np.sqrt(ms / (ms + EPS32)))) < 1e-12
    assert np.max(np.abs(rms_out - 1.0)) < 1e-5


def test_rmsnorm_exact_rows():
    # eps = 0 and rows of +-1 (mean square 1) or +-2 (mean square 4): r = 1 or 1/2 exactly
    g = synth.generator(6)
    s1 = g.choice([-1.0, 1.0], size=(4, 64))
    s2 = 2.0 * g.choice([-1.0, 1.0], size=(4, 64))
    gamma = g.standard_normal(64)
    assert np.array_equal(oracle.rmsnorm(s1, gamma, 0.0), s1 * gamma)
    assert np.array_equal(oracle.rmsnorm(s2, gamma, 0.0), (s2 * 0.5) * gamma)
    assert np.array_equal(oracle.rms_factor(s2, 0.0), np.full(4, 0.5))


def test_rmsnorm_scale_invariance_exact():
    g = synth.generator(7)
    X = g.standard_normal((8, 256))
    gamma = g.standard_normal(256)
    assert np.array_equal(oracle.rmsnorm(X, gamma, 0.0), oracle.rmsnorm(2.0 * X, gamma, 0.0))


def test_rmsnorm_matches_torch_rms_norm():
    g = synth.generator(8)
    X = g.standard_normal((16, 384)) * 3.0
    gamma = 1.0 + 0.1 * g.standard_normal(384)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(X), (384,), torch.from_numpy(gamma), EPS32).numpy()
    assert np.max(np.abs(oracle.rmsnorm(X, gamma, EPS32) - ref)) < 1e-13


def test_rmsnorm_eps_inside_root():
    e = _golden("rmsnorm_eps.txt")
    assert e["placement"] == "inside_root"
    X = np.full((1, 4), 1e-3)  # mean square 1e-6: eps matters at this scale
    eps = float(e["eps"])
    r = oracle.rms_factor(X, eps)[0]
    assert abs(r - 1.0 / math.sqrt(1e-6 + eps)) < 1e-9 * r
    assert abs(r - 1.0 / (math.sqrt(1e-6) + eps)) > 1.0  # eps outside the root differs a lot


def test_rmsnorm_linear_equals_normalise_then_matmul():
    g = synth.generator(9)
    X = g.standard_normal((12, 64))
    gamma = 1.0 + 0.1 * g.standard_normal(64)
    W = g.standard_normal((64, 40))
    xn = torch.nn.functional.rms_norm(torch.from_numpy(X), (64,), torch.from_numpy(gamma), EPS32).numpy()
    ref = xn @ W
    got = oracle.rmsnorm_gemm(X, gamma, EPS32, W)
    assert np.max(np.abs(got - ref)) < 1e-12 * np.max(np.abs(ref))


# --------------------------------------------------------------------------
# SwiGLU FFN
# --------------------------------------------------------------------------

def test_swiglu_gate_and_up_are_not_swapped():
    g = synth.generator(10)
    K = 32
    X = g.standard_normal((5, K))
    gamma = np.ones(K)
    H = oracle.rmsnorm_swiglu(X, gamma, EPS32, np.eye(K), 2.0 * np.eye(K))
    xn = torch.nn.functional.rms_norm(torch.from_numpy(X), (K,), None, EPS32).numpy()
    want = (xn * sp.expit(xn)) * (2.0 * xn)  # silu(gate) * up, gate = xn, up = 2 xn
    assert np.max(np.abs(H - want)) < 1e-13
    swapped = (2.0 * xn * sp.expit(2.0 * xn)) * xn
    assert np.max(np.abs(H - swapped)) > 1e-2


def test_swiglu_ffn_identity_down_projection():
    g = synth.generator(11)
    K = 16
    X = g.standard_normal((3, K))
    gamma = 1.0 + 0.1 * g.standard_normal(K)
    Wg = g.standard_normal((K, K))
    Wu = g.standard_normal((K, K))
    b = g.standard_normal(K)
    H = oracle.rmsnorm_swiglu(X, gamma, EPS32, Wg, Wu)
    Y = oracle.swiglu_ffn(X, gamma, EPS32, Wg, Wu, np.eye(K), b)
    assert np.array_equal(Y, H + b + X)


# --------------------------------------------------------------------------
# Brute force on tiny shapes (independent pure-Python implementation)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 7), (3, 7, 16), (7, 17, 3), (16, 16, 64), (17, 2, 64)])
@pytest.mark.parametrize("act_kind", ["none", "relu", "gelu_tanh", "silu"])
def test_brute_force_gemm_epilogue(M, N, K, act_kind):
    g = synth.generator(M * 10007 + N * 101 + K)
    A = g.standard_normal((M, K))
    W = g.standard_normal((K, N))
    b = g.standard_normal(N)
    R = g.standard_normal((M, N))
    for bias, res in ((None, None), (b, None), (b, R), (None, R)):
        want = np.array(brute.gemm_epilogue(A.tolist(), W.tolist(),
                                            None if bias is None else bias.tolist(),
                                            None if res is None else res.tolist(), act_kind))
        got = oracle.gemm_epilogue(A, W, bias, res, act_kind)
        assert np.max(np.abs(got - want)) < 1e-12 * max(1.0, np.max(np.abs(want)))


def test_brute_force_worked_example_shape():
    # The deplodock post walks x (16, 64) through a matmul with w (64, 16) and a ReLU.
    g = synth.generator(12)
    x = g.standard_normal((16, 64))
    w = g.standard_normal((64, 16))
    want = np.array(brute.gemm_epilogue(x.tolist(), w.tolist(), None, None, "relu"))
    got = oracle.gemm_epilogue(x, w, None, None, "relu")
    assert np.max(np.abs(got - want)) < 1e-12


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (3, 5, 16), (7, 9, 64)])
@pytest.mark.parametrize("act_kind", ["none", "gelu_tanh"])
def test_brute_force_rmsnorm_gemm_and_swiglu(M, N, K, act_kind):
    g = synth.generator(M + 1000 * K)
    X = g.standard_normal((M, K))
    gamma = 1.0 + 0.1 * g.standard_normal(K)
    W = g.standard_normal((K, N))
    W2 = g.standard_normal((K, N))
    b = g.standard_normal(N)
    want = np.array(brute.rmsnorm_gemm(X.tolist(), gamma.tolist(), EPS32, W.tolist(), b.tolist(), act_kind))
    got = oracle.rmsnorm_gemm(X, gamma, EPS32, W, b, act_kind)
    assert np.max(np.abs(got - want)) < 1e-12 * max(1.0, np.max(np.abs(want)))
    wantH = np.array(brute.rmsnorm_swiglu(X.tolist(), gamma.tolist(), EPS32, W.tolist(), W2.tolist()))
    gotH = oracle.rmsnorm_swiglu(X, gamma, EPS32, W, W2)
    assert np.max(np.abs(gotH - wantH)) < 1e-12 * max(1.0, np.max(np.abs(wantH)))


# --------------------------------------------------------------------------
# Synthetic-input plumbing shared by both sides
# --------------------------------------------------------------------------

def test_synth_rounding_matches_torch_casts():
    g = synth.generator(13)
    x = g.standard_normal(100000) * 10.0
    # fp16: correctly rounded from float64 -- no representable neighbour is closer,
    # and ties go to the even significand
    f16 = synth.to_bits(x, synth.F16)
    a = synth.widen(f16, synth.F16)
    h = f16.view(np.float16)
    up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h, np.float16(-np.inf)).astype(np.float64)
    assert np.all(np.abs(x - a) <= np.abs(x - up)) and np.all(np.abs(x - a) <= np.abs(x - dn))
    tie = (np.abs(x - a) == np.abs(x - up)) | (np.abs(x - a) == np.abs(x - dn))
    assert np.all((f16[tie] & 1) == 0)
    # agrees with torch's cast wherever the float32 detour of torch does not double-round
    t = torch.from_numpy(x).to(torch.float16).double().numpy()
    assert np.mean(a == t) > 0.999
    # bf16: float64 -> float32 -> bf16, both nearest-even; torch's float32 -> bf16 cast is the same
    bf = synth.to_bits(x, synth.BF16)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(synth.widen(bf, synth.BF16), want)


def test_synth_is_seeded_and_ordered():
    a = synth.rmsnorm_linear(M=4, D=64, N=32)
    b = synth.rmsnorm_linear(M=4, D=64, N=32)
    for k in a:
        assert np.array_equal(a[k], b[k])
    c = synth.decode_rmsnorm_linear(B=4, D=64)
    # decode draws W first: its X differs from the prefill draw with the same seed
    assert not np.array_equal(a["X"], c["X"])
    gam = synth.widen(a["gamma"], synth.F16)
    assert abs(gam.mean() - 1.0) < 0.1 and 0.03 < gam.std() < 0.3


# --------------------------------------------------------------------------
# LayerNorm -> GEMM ("llm-fusion-compiler" pattern table: layernorm_gemm)
# --------------------------------------------------------------------------

def test_layernorm_matches_torch_layer_norm():
    # torch.nn.functional.layer_norm in float64: mean, biased variance, eps
    # inside the root, then gamma and beta (an unbiased variance or eps outside
    # the root would differ by far more than 1e-12)
    g = synth.generator(51)
    for M, K in ((7, 40), (33, 257), (4, 4096)):
        X = g.standard_normal((M, K)) * 3.0 + g.standard_normal((M, 1)) * 5.0
        gamma = 1.0 + 0.1 * g.standard_normal(K)
        beta = 0.1 * g.standard_normal(K)
        for eps in (EPS32, 0.0, 1e-2):
            ref = torch.nn.functional.layer_norm(torch.from_numpy(X), (K,), torch.from_numpy(gamma),
                                                 torch.from_numpy(beta), eps).numpy()
            assert np.allclose(oracle.layernorm(X, gamma, eps, beta), ref, rtol=1e-12, atol=1e-12)
        ref = torch.nn.functional.layer_norm(torch.from_numpy(X), (K,), torch.from_numpy(gamma), None, EPS32).numpy()
        assert np.allclose(oracle.layernorm(X, gamma, EPS32), ref, rtol=1e-12, atol=1e-12)


def test_layernorm_closed_form_moments():
    # gamma = 1, beta = 0: every output row has mean 0 and variance
    # var / (var + eps), i.e. exactly 1 with eps = 0
    g = synth.generator(52)
    X = g.standard_normal((9, 300)) * 2.0 + 7.0
    for eps in (0.0, 0.5):
        Y = oracle.layernorm(X, np.ones(300), eps)
        var = X.var(axis=1)
        assert np.allclose(Y.mean(axis=1), 0.0, atol=1e-13)
        assert np.allclose(Y.var(axis=1), var / (var + eps), rtol=1e-12)


def test_layernorm_shift_and_scale_invariance():
    # LayerNorm(a x + c) == LayerNorm(x) for a > 0 and per-row constants c (eps = 0)
    g = synth.generator(53)
    X = g.standard_normal((6, 128))
    gamma, beta = 1.0 + 0.1 * g.standard_normal(128), g.standard_normal(128)
    base = oracle.layernorm(X, gamma, 0.0, beta)
    moved = oracle.layernorm(4.0 * X + g.standard_normal((6, 1)) * 100.0, gamma, 0.0, beta)
    assert np.allclose(moved, base, rtol=1e-10, atol=1e-10)


def test_layernorm_of_zero_mean_rows_is_rmsnorm():
    # rows built from +-v pairs have mean exactly 0, where LayerNorm (beta = 0)
    # and RMSNorm share one definition; rmsnorm is pinned to torch separately
    g = synth.generator(54)
    half = g.standard_normal((5, 64))
    X = np.concatenate([half, -half], axis=1)
    gamma = 1.0 + 0.1 * g.standard_normal(128)
    assert np.allclose(oracle.layernorm(X, gamma, EPS32), oracle.rmsnorm(X, gamma, EPS32), rtol=1e-13, atol=1e-15)


def test_layernorm_gemm_identity_weight_and_numpy():
    g = synth.generator(55)
    X = g.standard_normal((12, 64)) + 3.0
    gamma, beta = 1.0 + 0.1 * g.standard_normal(64), 0.1 * g.standard_normal(64)
    xh = oracle.layernorm(X, gamma, EPS32, beta)
    assert np.array_equal(oracle.layernorm_gemm(X, gamma, EPS32, np.eye(64), beta), xh)
    W = g.standard_normal((64, 40)) / 8.0
    b = 0.1 * g.standard_normal(40)
    assert np.allclose(oracle.layernorm_gemm(X, gamma, EPS32, W, beta, b, "none"), xh @ W + b, rtol=1e-12,
                       atol=1e-12)


@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (3, 7, 16), (16, 16, 64), (17, 9, 24)])
@pytest.mark.parametrize("act_kind", ["none", "relu", "gelu_tanh", "silu"])
def test_brute_force_layernorm_gemm(M, N, K, act_kind):
    g = synth.generator(M * 100 + N * 10 + K)
    X = g.standard_normal((M, K)) * 2.0 + 1.5
    gamma, beta = 1.0 + 0.1 * g.standard_normal(K), 0.1 * g.standard_normal(K)
    W = g.standard_normal((K, N)) / math.sqrt(K)
    b = 0.1 * g.standard_normal(N)
    want = brute.layernorm_gemm(X.tolist(), gamma.tolist(), EPS32, W.tolist(), beta.tolist(), b.tolist(), act_kind)
    got = oracle.layernorm_gemm(X, gamma, EPS32, W, beta, b, act_kind)
    assert np.allclose(got, np.array(want), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Prologue bias: act((x + b) @ W + bias) + R (deplodock post, Loop IR example)
# --------------------------------------------------------------------------

def test_prologue_bias_worked_example_shape():
    # the page's example relu((x + bias) @ w): x (16, 64), bias (64,), w (64, 16)
    g = synth.generator(56)
    x, ab, w = g.standard_normal((16, 64)), g.standard_normal(64), g.standard_normal((64, 16))
    want = brute.prologue_bias_gemm(x.tolist(), ab.tolist(), w.tolist(), None, None, "relu")
    got = oracle.prologue_bias_gemm(x, ab, w, act_kind="relu")
    assert np.allclose(got, np.array(want), rtol=1e-12, atol=1e-12)
    # and relu applies after the reduction, not to x + bias: numpy's matmul
    assert np.allclose(got, np.maximum((x + ab) @ w, 0.0), rtol=1e-12, atol=1e-12)


def test_prologue_bias_is_linear_in_the_bias():
    # (A + 1 b) W = A W + 1 (b W): numpy matmul on both terms
    g = synth.generator(57)
    A, ab, W = g.standard_normal((20, 48)), g.standard_normal(48), g.standard_normal((48, 24))
    bias, R = g.standard_normal(24), g.standard_normal((20, 24))
    got = oracle.prologue_bias_gemm(A, ab, W, bias, R, "none")
    assert np.allclose(got, A @ W + (ab @ W)[None, :] + bias + R, rtol=1e-12, atol=1e-12)


def test_prologue_bias_identity_weight_and_integers():
    g = synth.generator(58)
    A = g.integers(-3, 4, (10, 32)).astype(np.float64)
    ab = g.integers(-3, 4, 32).astype(np.float64)
    # W = I: Y = act(A + b + bias) + R elementwise, exactly
    bias = g.integers(-5, 6, 32).astype(np.float64)
    R = g.integers(-5, 6, (10, 32)).astype(np.float64)
    assert np.array_equal(oracle.prologue_bias_gemm(A, ab, np.eye(32), bias, R, "relu"),
                          np.maximum(A + ab + bias, 0.0) + R)
    # small integers: exact, equal to int64 matmul
    W = g.integers(-2, 3, (32, 17))
    want = (A.astype(np.int64) + ab.astype(np.int64)) @ W
    assert np.array_equal(oracle.prologue_bias_gemm(A, ab, W.astype(np.float64)), want.astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (5, 7, 16), (17, 9, 24)])
@pytest.mark.parametrize("act_kind", ["none", "gelu_tanh", "silu"])
def test_brute_force_prologue_bias(M, N, K, act_kind):
    g = synth.generator(M * 97 + N * 13 + K)
    A, ab, W = g.standard_normal((M, K)), g.standard_normal(K), g.standard_normal((K, N)) / math.sqrt(K)
    b, R = 0.1 * g.standard_normal(N), g.standard_normal((M, N))
    want = brute.prologue_bias_gemm(A.tolist(), ab.tolist(), W.tolist(), b.tolist(), R.tolist(), act_kind)
    assert np.allclose(oracle.prologue_bias_gemm(A, ab, W, b, R, act_kind), np.array(want), rtol=1e-12,
                       atol=1e-12)
