"""The tuner on the device (needs an MI355X): candidates are timed, the
fastest is registered and cached, the HIP runtime's resource report of every
candidate's kernel is within gfx950's limits, and the tuned plan's output
matches the oracle."""
import numpy as np
import pytest

import gemm_epilogue_fuse_amd as lf
import oracle
import synth
from gemm_epilogue_fuse_amd import tuner
from parity_util import EPS, EPS32, assert_close, dev_t, say, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def clean_table():
    lf.set_plan(None)
    lf.lib().fuse_tune_clear()
    yield
    lf.lib().fuse_tune_clear()


def test_every_candidate_kernel_is_within_the_hardware_limits():
    for op, (M, N, K) in ((0, (512, 4096, 4096)), (1, (32, 4096, 4096)), (2, (512, 1024, 1024)),
                          (3, (256, 512, 520))):
        for c in tuner.candidates(op, M, N, K):
            tuner.set_tuned(op, M, N, K, lf.F16, c)
            res = tuner.resources(op, M, N, K, lf.F16)
            say("resources", op, M, N, K, c, res)
            assert tuner.within_limits(res), (c, res)
    tuner.set_tuned(op, M, N, K, lf.F16, None)


@pytest.mark.parametrize("op,M,N,K", [(1, 512, 4096, 4096), (1, 32, 4096, 4096), (0, 1024, 4096, 4096)])
def test_tune_registers_and_caches_the_fastest(tmp_path, op, M, N, K):
    path = str(tmp_path / "tune.json")
    r = tuner.tune(op, M, N, K, lf.F16, launches=10, path=path, max_candidates=8)
    say("tuned", op, M, N, K, r["plan"], r["us"], "static", r["default_plan"], r["default_us"])
    assert r["source"] == "measured" and r["plan"] in r["candidates"]
    assert r["us"] == min(r["candidates"].values())
    assert lf.plan_name(op, M, N, K) == r["plan"]
    lf.lib().fuse_tune_clear()
    assert tuner.load_cache(path) == 1 and lf.plan_name(op, M, N, K) == r["plan"]
    # the tuned plan computes the operator
    if op == 1:
        d = synth.rmsnorm_linear(M=M, D=K, N=N, seed=5)
        t = {k: dev_t(v, synth.F16) for k, v in d.items()}
        x = {k: synth.widen(v, synth.F16) for k, v in d.items()}
        got = to64(lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], EPS))
        want = oracle.rmsnorm_gemm(x["X"], x["gamma"], EPS32, x["W"])
    else:
        d = synth.gemm_epilogue_sweep(M, N, K, seed=5)
        t = {k: dev_t(v, synth.F16) for k, v in d.items()}
        x = {k: synth.widen(v, synth.F16) for k, v in d.items()}
        got = to64(lf.gemm_epilogue(t["A"], t["W"], t["bias"], None, "gelu_tanh"))
        want = oracle.gemm_epilogue(x["A"], x["W"], x["bias"], None, "gelu_tanh")
    assert np.all(np.isfinite(got))
    assert_close(got, want, "tuned plan %s" % r["plan"])
