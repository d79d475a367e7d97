#!/usr/bin/env python3
"""Benchmark of the fused GEMM + epilogue and RMSNorm -> Linear kernels on one MI355X.

Default run: one JSON line on stdout.  Its headline is the fused RMSNorm ->
Linear workload X[512,4096] fp16 -> RMSNorm(gamma, eps=1e-6) -> . W[4096,4096],
no bias, no activation ("LLMBoost", benchmark results: the [512,4096] x
[4096,4096] fp16 shape).  One step = one fused call over one batch of
resident inputs.  ``workloads`` in the same line carries every other
workload at its full size: the 64x256x256 GEMM + bias + GeLU, the GEMM +
bias + activation sweep (M = 512..4096, N = K = 4096) with its SiLU, ReLU and
residual variants, the bf16 SwiGLU FFN block (both kernels and their sum),
LayerNorm -> Linear and the input-bias GEMM (the adjacent prologue fusions),
and the decode-shaped RMSNorm -> Linear cells (B x D, fp16 and bf16).  Each
carries its roofline fields and, beside it, the same computation unfused
through torch (rms_norm, hipBLASLt matmul, separate elementwise kernels),
timed the same way ("llm-fusion-compiler", benchmark table: generated kernel
against the vendor library; "LLMBoost", benchmark results and speedup across
shapes: unfused against fused).

Timing.  Every workload is timed as a HIP graph of back-to-back calls over
enough independent input sets that consecutive calls cannot hit in the 256 MB
last-level cache (the layer-after-layer situation of a model), replayed on
one stream; wall clock and HIP events on that stream bracket the same replay.
The headline's graph holds exactly --steps calls.

    python bench.py [--steps K] [--warmup W] [--only NAME] [--no-cpu] [--no-sweep]

``--only`` keeps the workloads whose name contains NAME (for profiling one
kernel at a time; the headline is always timed).  ``--calibrate-copy`` runs a
plain device copy of known size for scaling hardware traffic counters.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused GEMM+epilogue TFLOP/s & %MFMA peak; RMSNorm→Linear latency, HBM GB/s"
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
ROTATE_BYTES = 640 << 20    # footprint of the rotating input sets (> 256 MB MALL)
EPS = 1e-6
# The pages' own figure for this exact workload: 0.208 ms fused on an NVIDIA A30
# ("LLMBoost", benchmark results).  Context only (other hardware).
PAGE_A30_MS = 0.208
HEADLINE = "rmsnorm_linear_512x4096x4096_fp16"

# Every device source compiled into libfuse: the stored hardware-counter
# summaries are used only while these hash to the value recorded with them.
CSRC = "gemm_epilogue_fuse_amd/csrc/"
KERNEL_SOURCES = [CSRC + f for f in (
    "gemm_fused.hip", "kernels.h", "k_dma_square.hip", "k_dma_wide.hip", "k_dma_pro.hip", "k_reg.hip", "k_small.hip",
    "kernel_dma.h", "kernel_reg.h", "common.h", "kernel_decode.h", "kernel_strip.h", "kernel_wstrip.h",
    "launch.h")]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- timing

# Untimed launches before the timed replay, long enough for the GPU clocks to
# leave their idle state (a few ms of launches after an idle host phase
# measured about 10% slow).
SETTLE_S = 0.3


def capture(calls, stream):
    """A HIP graph of calls[i](stream) for every i, captured on `stream`."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c(stream)
    return g


def time_graph(call_on, nsets, launches, warmup, settle_s=None, replays=1):
    """Time `launches` calls call_on(i % nsets, stream) captured in one HIP graph.

    The calls first run eagerly (settle_s seconds, then `warmup` more), which
    also creates any per-stream library state before capture.  Then the graph
    is replayed `replays` times, bracketed by torch.cuda.synchronize(), a wall
    clock and HIP events recorded on the replay stream.  Returns (wall ms per
    call, event ms per call)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    t_end = time.perf_counter() + (SETTLE_S if settle_s is None else settle_s)
    i = 0
    with torch.cuda.stream(s):
        while True:
            for _ in range(max(warmup, nsets)):
                call_on(i % nsets, s)
                i += 1
            s.synchronize()
            if time.perf_counter() >= t_end:
                break
    g = capture([(lambda st, j=j: call_on(j % nsets, st)) for j in range(launches)], s)
    with torch.cuda.stream(s):
        g.replay()  # the first replay uploads the graph
        s.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(s)
        for _ in range(replays):
            g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / (launches * replays)
    dev = e0.elapsed_time(e1) / (launches * replays)
    del g
    return wall, dev


def launch_floor_us(launches=200):
    """Device time per call of a one-element device op in a replayed HIP graph:
    the floor under any call's latency."""
    import torch
    x = torch.zeros(1, device="cuda:0")
    _, dev = time_graph(lambda i, st: x.add_(1.0), 1, launches, 20, settle_s=0.0, replays=5)
    return round(dev * 1e3, 3)


def n_sets(bytes_per_set):
    return max(2, min(64, (ROTATE_BYTES + bytes_per_set - 1) // bytes_per_set))


def result_fields(dev_ms, flops, alg_bytes):
    tflops = flops / (dev_ms * 1e-3) / 1e12
    gbs = alg_bytes / (dev_ms * 1e-3) / 1e9
    t_mfma = flops / (PEAK_MFMA_TFLOPS * 1e12)
    t_hbm = alg_bytes / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    return {
        "latency_us": round(dev_ms * 1e3, 3),
        "tflops": round(tflops, 2),
        "mfma_frac": round(tflops / PEAK_MFMA_TFLOPS, 4),
        "hbm_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "roof_bound": bound,
        "roof_us": round(max(t_mfma, t_hbm) * 1e6, 3),
    }


# ----------------------------------------------------------------------------- traffic counters

def read_traffic(name):
    """Bytes per launch between the L2 and the memory fabric (L2 misses, served
    by the last-level cache or HBM) from the committed rocprofv3 counter
    summary, or None if absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#") and ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_hash():
        return None
    try:
        return float(vals["l2_fabric_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(min_seconds=10.0):
    """The fp64 oracle, as it stands, on the headline workload (whole 512x4096x4096
    problem, repeated until ~min_seconds of CPU work), in TFLOP/s."""
    import numpy as np
    import oracle
    import synth
    d = synth.rmsnorm_linear(M=512, D=4096, N=4096, seed=0)
    x = {k: synth.widen(v, synth.F16) for k, v in d.items()}
    eps32 = float(np.float32(EPS))
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    oracle.rmsnorm_gemm(x["X"][:8], x["gamma"], eps32, x["W"])  # build + warm
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.rmsnorm_gemm(x["X"], x["gamma"], eps32, x["W"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= 200:
            break
    per = el / reps
    return {"value": round(2.0 * 512 * 4096 * 4096 / per / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": "whole 512x4096x4096 fp16 RMSNorm->Linear workload in fp64, %d repetitions, %.2f s each"
                      % (reps, per)}


# ----------------------------------------------------------------------------- workloads
#
# A workload: its inputs (drawn once with the seeded generators, then cloned
# into rotating sets on the device), the fused call through the C ABI with
# pre-marshalled pointers (what a native caller does), and the same
# computation unfused through torch.

class Workload:
    def __init__(self, name, dtype, flops, alg_bytes, make, fused, unfused, plan, extra=None):
        self.name, self.dtype, self.flops, self.alg_bytes = name, dtype, flops, alg_bytes
        self.make, self.fused, self.unfused, self.plan = make, fused, unfused, plan
        self.extra = extra or {}


def _dev(bits, dt):
    import synth
    return synth.to_torch(bits, dt, "cuda:0")


def _sets(base, bytes_per_set, outputs):
    """Rotating input sets: set 0 is `base`, the others device clones; each set
    gets its own output buffers from outputs()."""
    sets = []
    for i in range(n_sets(bytes_per_set)):
        t = dict(base) if i == 0 else {k: v.clone() for k, v in base.items()}
        t.update(outputs())
        sets.append(t)
    return sets


def _code(lf, dt):
    import synth
    return lf.BF16 if dt == synth.BF16 else lf.F16


def gemm_workload(lf, name, M, N, K, act, resid, dt, draw):
    import torch
    import torch.nn.functional as F
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    alg = (M * K + K * N + N + M * N * (2 if resid else 1)) * 2
    code = _code(lf, dt)
    L = lf.lib()
    actc = lf.ACT[act]

    def make():
        d = draw()
        base = {k: _dev(v, dt) for k, v in d.items()}
        return _sets(base, alg, lambda: {"Y": torch.empty((M, N), dtype=tdt, device="cuda:0")})

    def fused(s):
        args = (s["A"].data_ptr(), s["W"].data_ptr(), s["bias"].data_ptr(),
                s["R"].data_ptr() if resid else None, s["Y"].data_ptr())

        def call(st):
            rc = L.fuse_gemm_epilogue(*args, M, N, K, actc, code, ctypes.c_void_p(st.cuda_stream))
            if rc:
                raise lf.FuseError(rc, "fuse_gemm_epilogue")
        return call

    def unfused(s):
        A, W, b = s["A"], s["W"], s["bias"]
        R = s.get("R")

        def call(st):
            z = torch.addmm(b, A, W)
            if act == "gelu_tanh":
                z = F.gelu(z, approximate="tanh")
            elif act == "silu":
                z = F.silu(z)
            elif act == "relu":
                z = F.relu(z)
            if R is not None:
                z = z + R
            return z
        return call
    return Workload(name, dt, 2.0 * M * N * K, alg, make, fused, unfused, lf.plan_name(0, M, N, K, code))


def rms_workload(lf, name, M, D, N, dt, draw):
    import torch
    import torch.nn.functional as F
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    alg = (M * D + D + D * N + M * N) * 2
    code = _code(lf, dt)
    L = lf.lib()
    eps = ctypes.c_float(EPS)

    def make():
        d = draw()
        base = {k: _dev(v, dt) for k, v in d.items()}
        return _sets(base, alg, lambda: {"Y": torch.empty((M, N), dtype=tdt, device="cuda:0")})

    def fused(s):
        args = (s["X"].data_ptr(), s["gamma"].data_ptr(), eps, s["W"].data_ptr(), None, s["Y"].data_ptr())

        def call(st):
            rc = L.fuse_rmsnorm_gemm(*args, M, N, D, 0, code, ctypes.c_void_p(st.cuda_stream))
            if rc:
                raise lf.FuseError(rc, "fuse_rmsnorm_gemm")
        return call

    def unfused(s):
        X, g, W = s["X"], s["gamma"], s["W"]
        return lambda st: torch.matmul(F.rms_norm(X, (D,), g, EPS), W)
    return Workload(name, dt, 2.0 * M * N * D, alg, make, fused, unfused, lf.plan_name(1, M, N, D, code))


def layernorm_workload(lf, name, M, D, N, act, dt):
    """LayerNorm -> Linear + bias + activation (the layernorm_gemm pattern)."""
    import torch
    import torch.nn.functional as F
    import numpy as np
    import synth
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    alg = (M * D + 2 * D + D * N + N + M * N) * 2
    code = _code(lf, dt)
    L = lf.lib()
    actc = lf.ACT[act]
    eps = ctypes.c_float(1e-5)

    def make():
        g = synth.generator(0)
        X = synth.normal(g, (M, D), 1.0)
        fields = [("X", X), ("gamma", synth.normal(g, (D,), 0.1, 1.0)), ("beta", synth.normal(g, (D,), 0.1)),
                  ("W", synth.normal(g, (D, N), 1.0 / np.sqrt(D))), ("bias", synth.normal(g, (N,), 0.1))]
        base = {k: _dev(synth.to_bits(v, dt), dt) for k, v in fields}
        return _sets(base, alg, lambda: {"Y": torch.empty((M, N), dtype=tdt, device="cuda:0")})

    def fused(s):
        args = (s["X"].data_ptr(), s["gamma"].data_ptr(), s["beta"].data_ptr(), eps, s["W"].data_ptr(),
                s["bias"].data_ptr(), s["Y"].data_ptr())

        def call(st):
            rc = L.fuse_layernorm_gemm(*args, M, N, D, actc, code, ctypes.c_void_p(st.cuda_stream))
            if rc:
                raise lf.FuseError(rc, "fuse_layernorm_gemm")
        return call

    def unfused(s):
        X, g, be, W, b = s["X"], s["gamma"], s["beta"], s["W"], s["bias"]
        return lambda st: F.gelu(torch.addmm(b, F.layer_norm(X, (D,), g, be, 1e-5), W), approximate="tanh")
    return Workload(name, dt, 2.0 * M * N * D, alg, make, fused, unfused, lf.plan_name(3, M, N, D, code))


def prologue_bias_workload(lf, name, M, K, N, act, dt):
    """act((A + b) W + bias): the input bias added inside the reduction."""
    import torch
    import torch.nn.functional as F
    import synth
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    alg = (M * K + K + K * N + N + M * N) * 2
    code = _code(lf, dt)
    L = lf.lib()
    actc = lf.ACT[act]

    def make():
        g = synth.generator(0)
        fields = [("A", synth.normal(g, (M, K), 1.0)), ("abias", synth.normal(g, (K,), 1.0)),
                  ("W", synth.normal(g, (K, N), 1.0 / 64.0)), ("bias", synth.normal(g, (N,), 0.1))]
        base = {k: _dev(synth.to_bits(v, dt), dt) for k, v in fields}
        return _sets(base, alg, lambda: {"Y": torch.empty((M, N), dtype=tdt, device="cuda:0")})

    def fused(s):
        args = (s["A"].data_ptr(), s["abias"].data_ptr(), s["W"].data_ptr(), s["bias"].data_ptr(), None,
                s["Y"].data_ptr())

        def call(st):
            rc = L.fuse_gemm_prologue_bias(*args, M, N, K, actc, code, ctypes.c_void_p(st.cuda_stream))
            if rc:
                raise lf.FuseError(rc, "fuse_gemm_prologue_bias")
        return call

    def unfused(s):
        A, ab, W, b = s["A"], s["abias"], s["W"], s["bias"]
        return lambda st: F.gelu(torch.addmm(b, A + ab, W), approximate="tanh")
    return Workload(name, dt, 2.0 * M * N * K, alg, make, fused, unfused, lf.plan_name(4, M, N, K, code))


def swiglu_workloads(lf, M, D, F_):
    """The bf16 SwiGLU FFN block as its two fused kernels, and their sum."""
    import torch
    import torch.nn.functional as F
    import synth
    L = lf.lib()
    code = lf.BF16
    eps = ctypes.c_float(EPS)
    b1 = (M * D + D + 2 * D * F_ + M * F_) * 2
    b2 = (M * F_ + F_ * D + D + 2 * M * D) * 2
    shared = {}

    def make():
        if "sets" not in shared:
            d = synth.swiglu_ffn(M=M, D=D, F=F_, seed=0)
            base = {k: _dev(v, synth.BF16) for k, v in d.items()}
            shared["sets"] = _sets(base, b1 + b2, lambda: {
                "H": torch.empty((M, F_), dtype=torch.bfloat16, device="cuda:0"),
                "Y": torch.empty((M, D), dtype=torch.bfloat16, device="cuda:0")})
        return shared["sets"]

    def k1(s):
        a = (s["X"].data_ptr(), s["gamma"].data_ptr(), eps, s["Wg"].data_ptr(), s["Wu"].data_ptr(),
             s["H"].data_ptr())

        def call(st):
            rc = L.fuse_rmsnorm_gemm_swiglu(*a, M, F_, D, code, ctypes.c_void_p(st.cuda_stream))
            if rc:
                raise lf.FuseError(rc, "fuse_rmsnorm_gemm_swiglu")
        return call

    def k2(s):
        a = (s["H"].data_ptr(), s["Wd"].data_ptr(), s["bias"].data_ptr(), s["X"].data_ptr(), s["Y"].data_ptr())

        def call(st):
            rc = L.fuse_gemm_epilogue(*a, M, D, F_, 0, code, ctypes.c_void_p(st.cuda_stream))
            if rc:
                raise lf.FuseError(rc, "fuse_gemm_epilogue")
        return call

    def block(s):
        c1, c2 = k1(s), k2(s)

        def call(st):
            c1(st)
            c2(st)
        return call

    def u1(s):
        X, g, Wg, Wu = s["X"], s["gamma"], s["Wg"], s["Wu"]

        def call(st):
            xn = F.rms_norm(X, (D,), g, EPS)
            return F.silu(torch.matmul(xn, Wg)) * torch.matmul(xn, Wu)
        return call

    def u2(s):
        H, Wd, b, X = s["H"], s["Wd"], s["bias"], s["X"]
        return lambda st: torch.addmm(b, H, Wd) + X

    def ub(s):
        c1, c2 = u1(s), u2(s)
        Wd, b, X = s["Wd"], s["bias"], s["X"]
        return lambda st: torch.addmm(b, c1(st), Wd) + X

    f1, f2 = 4.0 * M * F_ * D, 2.0 * M * D * F_
    return [
        Workload("swiglu_k1_rmsnorm_gate_up_%dx%dx%d_bf16" % (M, F_, D), "bf16", f1, b1, make, k1, u1,
                 lf.plan_name(2, M, F_, D, code)),
        Workload("swiglu_k2_down_bias_residual_%dx%dx%d_bf16" % (M, D, F_), "bf16", f2, b2, make, k2, u2,
                 lf.plan_name(0, M, D, F_, code)),
        Workload("swiglu_ffn_block_%dx%dx%d_bf16" % (M, D, F_), "bf16", f1 + f2, b1 + b2, make, block, ub,
                 lf.plan_name(2, M, F_, D, code) + " + " + lf.plan_name(0, M, D, F_, code)),
    ]


def all_workloads(lf):
    import synth
    ws = [gemm_workload(lf, "gemm_bias_gelu_tanh_64x256x256_fp16", 64, 256, 256, "gelu_tanh", False, "f16",
                        lambda: synth.gemm_bias_gelu_small(seed=0))]
    for M, act, resid in [(512, "gelu_tanh", False), (1024, "gelu_tanh", False), (2048, "gelu_tanh", False),
                          (4096, "gelu_tanh", False), (4096, "silu", False), (4096, "relu", False),
                          (4096, "none", True)]:
        name = "gemm_bias_%s%s_%dx4096x4096_fp16" % ("residual" if resid else act, "", M)
        ws.append(gemm_workload(lf, name, M, 4096, 4096, act, resid, "f16",
                                lambda M=M, resid=resid: synth.gemm_epilogue_sweep(M, seed=0, residual=resid)))
    ws += swiglu_workloads(lf, 2048, 4096, 11008)
    # the adjacent prologue fusions: LayerNorm -> Linear and an input bias
    ws.append(layernorm_workload(lf, "layernorm_gemm_gelu_tanh_2048x4096x4096_fp16", 2048, 4096, 4096,
                                 "gelu_tanh", "f16"))
    ws.append(prologue_bias_workload(lf, "prologue_bias_gemm_gelu_tanh_4096x4096x4096_fp16", 4096, 4096, 4096,
                                     "gelu_tanh", "f16"))
    for dt in (synth.F16, synth.BF16):
        for D in (1024, 2048, 4096):
            for B in (1, 32, 128, 512, 1024):
                ws.append(rms_workload(lf, "decode_rmsnorm_linear_B%d_D%d_%s" % (B, D, dt), B, D, D, dt,
                                       lambda B=B, D=D, dt=dt: synth.decode_rmsnorm_linear(B, D, seed=0, dtype=dt)))
                ws[-1].extra["decode"] = True
    return ws


def measure(w, launches=40, warmup=5, floor=None):
    """Fused and unfused timings of one workload, as one record."""
    sets = w.make()
    fused = [w.fused(s) for s in sets]
    unfused = [w.unfused(s) for s in sets]
    nl = max(launches, len(sets))
    _, dev = time_graph(lambda i, st: fused[i](st), len(sets), nl, warmup, settle_s=0.05, replays=2)
    _, udev = time_graph(lambda i, st: unfused[i](st), len(sets), nl, warmup, settle_s=0.02, replays=2)
    rec = {"workload": w.name, "dtype": w.dtype, "plan": w.plan}
    rec.update(result_fields(dev, w.flops, w.alg_bytes))
    rec["unfused_latency_us"] = round(udev * 1e3, 3)
    rec["unfused"] = "torch: rms_norm / addmm and matmul (hipBLASLt) / separate elementwise kernels"
    rec["speedup_vs_unfused"] = round(udev / dev, 3)
    rec["rotating_input_sets"] = len(sets)
    if w.extra.get("decode") and floor is not None:
        rec["launch_floor_us"] = floor
        rec["below_launch_floor"] = rec["roof_us"] < floor
        rec["hbm_frac_cap"] = round(min(1.0, (w.alg_bytes / (PEAK_HBM_GBS * 1e9)) /
                                        max(w.flops / (PEAK_MFMA_TFLOPS * 1e12), w.alg_bytes / (PEAK_HBM_GBS * 1e9))), 4)
    return rec


# ----------------------------------------------------------------------------- main

def main():
    global SETTLE_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default=None, help="only the extra workloads whose name contains this")
    ap.add_argument("--no-sweep", action="store_true", help="headline only")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed launches before the headline's timed replay (0 under counter runs)")
    args = ap.parse_args()
    SETTLE_S = max(0.0, args.settle)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: libfuse runs its fused kernels on a single MI355X "
              "(there is no multi-GPU path); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_epilogue_fuse_amd as lf
    import synth
    if not os.path.exists(lf.LIB_PATH):
        from gemm_epilogue_fuse_amd import build
        build.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)
    log("device: %s, %d CUs, arch %s" % (props.name, props.multi_processor_count, getattr(props, "gcnArchName", "?")))

    if args.calibrate_copy:
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: %d bytes read + %d bytes written per launch, 5 launches" % (n, n))
        return

    # ---- headline: exactly --steps calls in one graph, replayed once
    M, D, N = 512, 4096, 4096
    hw = rms_workload(lf, HEADLINE, M, D, N, synth.F16,
                      lambda: synth.rmsnorm_linear(M=M, D=D, N=N, seed=0))
    sets = hw.make()
    calls = [hw.fused(s) for s in sets]
    wall_ms, dev_ms = time_graph(lambda i, st: calls[i](st), len(sets), args.steps, args.warmup)
    fields = result_fields(dev_ms, hw.flops, hw.alg_bytes)
    value = hw.flops / (wall_ms * 1e-3) / 1e12       # whole-job throughput over the timed region
    traffic = read_traffic("rmsnorm_linear_512x4096x4096_fp16.traffic.txt")
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(PAGE_A30_MS / wall_ms, 3),
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "M": M, "K": D, "N": N, "eps": EPS, "bias": None, "act": "none",
                   "seed": 0, "plan": hw.plan, "rotating_input_sets": len(sets), "clock_settle_s": SETTLE_S,
                   "parallelism": "none (1 GPU)"},
        "timing": "one HIP graph of exactly `steps` calls over the rotating input sets, replayed once; "
                  "value and ms_per_step from the wall clock, roofline from HIP events on the replay stream, "
                  "both around that same replay",
        "latency_us": fields["latency_us"],
        "hbm_gbs": fields["hbm_gbs"],
        "mfma_frac": fields["mfma_frac"],
        "hbm_frac": fields["hbm_frac"],
        "roofline": {"bound": "mfma", "achieved": fields["tflops"], "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": fields["mfma_frac"], "traffic": traffic,
                     "algorithmic_bytes": hw.alg_bytes, "algorithmic_flops": hw.flops,
                     "kernel": "gemm_dma_kernel (plan %s)" % hw.plan,
                     "kernel_source_sha256_16": kernel_hash()},
        "baseline_context": "0.208 ms fused on an NVIDIA A30 (page figure, other hardware); "
                            "vs_baseline = 0.208 ms / ms_per_step",
    }
    # the same work unfused through torch, over the same input sets, after the timed region
    ucalls = [hw.unfused(s) for s in sets]
    _, udev = time_graph(lambda i, st: ucalls[i](st), len(sets), max(40, len(sets)), 5, settle_s=0.02, replays=2)
    rec["unfused_latency_us"] = round(udev * 1e3, 3)
    rec["unfused"] = "torch: rms_norm, then matmul (hipBLASLt)"
    rec["speedup_vs_unfused"] = round(udev / dev_ms, 3)
    del calls, ucalls, sets
    log("headline: %.3f us per call (events), %.3f us (wall); unfused torch %.3f us" %
        (dev_ms * 1e3, wall_ms * 1e3, udev * 1e3))

    # ---- every other workload, fused and unfused
    if not args.no_sweep:
        floor = launch_floor_us()
        rec["launch_floor_us"] = floor
        out = []
        for w in all_workloads(lf):
            if args.only is not None and args.only not in w.name:
                continue
            r = measure(w, floor=floor)
            log(json.dumps(r))
            out.append(r)
            torch.cuda.empty_cache()
        rec["workloads"] = out

    if not args.no_cpu:
        log("timing the fp64 oracle on the host cores ...")
        rec["cpu_baseline"] = cpu_baseline()
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
