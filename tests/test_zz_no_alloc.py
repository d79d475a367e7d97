"""The allocation-free RMSNorm -> Linear entry point against the allocating one
(needs an MI355X).

fuse_rmsnorm_gemm_noalloc runs the same kernels as fuse_rmsnorm_gemm with the
split-K partials in a fixed per-device buffer instead of a hipMalloc'd
workspace, so its output must equal fuse_rmsnorm_gemm's bit for bit.  Two
calls in a row, the second smaller (the buffer keeps the first call's
contents), for split-K and non-split shapes; then calls captured into a HIP
graph and replayed several times with eager work in between.
"""
import ctypes

import numpy as np
import pytest

import gemm_epilogue_fuse_amd as lf
import synth
from parity_util import EPS, dev_t, say

pytestmark = pytest.mark.gpu

# (first call, second smaller call): M, K, N
PAIRS = [((512, 4096, 4096), (130, 2048, 1024)),   # 128x128 split-K, then the 64x128 split tile
         ((128, 4096, 4096), (1, 4096, 4096)),     # 64x128 split K 4, then small-M chunks
         ((32, 4096, 2048), (17, 1024, 520)),      # small-M chunks, then the whole-strip kernel
         ((1024, 2048, 4096), (512, 512, 1032))]   # no split, then a short split


def call_noalloc(X, g, W, Y, M, N, K, dtype, stream):
    L = lf.lib()
    code = lf.BF16 if dtype == synth.BF16 else lf.F16
    rc = L.fuse_rmsnorm_gemm_noalloc(X.data_ptr(), g.data_ptr(), ctypes.c_float(EPS), W.data_ptr(), None,
                                     Y.data_ptr(), M, N, K, 0, code, ctypes.c_void_p(stream))
    assert rc == 0, L.fuse_strerror(rc)


def inputs(M, K, N, dtype, seed):
    d = synth.rmsnorm_linear(M=M, D=K, N=N, seed=seed, dtype=dtype)
    return {k: dev_t(v, dtype) for k, v in d.items()}


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_allocating_entry_point(first, second, dtype):
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    for i, (M, K, N) in enumerate((first, second)):
        say("noalloc", dtype, M, K, N, lf.plan_name(1, M, N, K, lf.BF16 if dtype == synth.BF16 else lf.F16))
        t = inputs(M, K, N, dtype, seed=60 + i)
        want = lf.rmsnorm_gemm(t["X"], t["gamma"], t["W"], EPS)
        got = torch.full((M, N), float("nan"), dtype=want.dtype, device="cuda:0")
        call_noalloc(t["X"], t["gamma"], t["W"], got, M, N, K, dtype, stream)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (M, K, N)


def test_noalloc_under_graph_capture():
    """Captured on a fresh stream with no eager call on it, replayed several
    times with eager calls of other shapes in between: every replay equals
    the allocating entry point's eager result."""
    import torch
    dt = synth.F16
    shapes = [(512, 4096, 4096), (1, 4096, 4096)]
    sets = [inputs(M, K, N, dt, seed=70 + j) for j, (M, K, N) in enumerate(shapes)]
    want = [lf.rmsnorm_gemm(s["X"], s["gamma"], s["W"], EPS) for s in sets]
    outs = [torch.full_like(w, float("nan")) for w in want]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    say("noalloc graph capture", shapes)
    with torch.cuda.graph(g, stream=s):
        for (M, K, N), t, o in zip(shapes, sets, outs):
            call_noalloc(t["X"], t["gamma"], t["W"], o, M, N, K, dt, s.cuda_stream)
    other = inputs(128, 2048, 2048, dt, seed=79)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o.view(torch.int16), w.view(torch.int16)), rep
        # eager work in between, on the same scratch
        y = torch.empty((128, 2048), dtype=torch.float16, device="cuda:0")
        call_noalloc(other["X"], other["gamma"], other["W"], y, 128, 2048, 2048, dt,
                     torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(y, lf.rmsnorm_gemm(other["X"], other["gamma"], other["W"], EPS))
