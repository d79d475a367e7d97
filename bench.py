#!/usr/bin/env python3
"""Benchmark of the fused RMSNorm -> Linear / GEMM + epilogue kernels on one MI355X.

Default run (one JSON line on stdout): the fused RMSNorm -> Linear workload
X[512,4096] fp16 -> RMSNorm(gamma, eps=1e-6) -> . W[4096,4096], no bias, no
activation ("LLMBoost", benchmark results: the [512,4096] x [4096,4096] fp16
shape).  One step = one fused call over one batch of resident inputs.  The
inputs rotate over enough independent sets that consecutive steps cannot hit
in the 256 MB last-level cache (the layer-after-layer situation of a model).

    python bench.py [--steps K] [--warmup W] [--sweep] [--no-cpu]

``--sweep`` also prints one JSON line per extra workload to stderr (the
GEMM + bias + activation sweep, the SwiGLU FFN block and the decode-shaped
RMSNorm -> Linear cells).  ``--calibrate-copy`` runs a plain device copy of
known size for scaling hardware traffic counters.
"""
from __future__ import annotations

import argparse
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

# Every device source compiled into libfuse: the stored HBM-traffic counters
# are used only while these hash to the value recorded with them.
KERNEL_SOURCES = ["gemm_epilogue_fuse_amd/csrc/gemm_fused.hip", "gemm_epilogue_fuse_amd/csrc/kernels.h",
                  "gemm_epilogue_fuse_amd/csrc/k_dma_square.hip", "gemm_epilogue_fuse_amd/csrc/k_dma_wide.hip",
                  "gemm_epilogue_fuse_amd/csrc/k_reg.hip", "gemm_epilogue_fuse_amd/csrc/k_small.hip",
                  "gemm_epilogue_fuse_amd/csrc/kernel_dma.h",
                  "gemm_epilogue_fuse_amd/csrc/kernel_reg.h", "gemm_epilogue_fuse_amd/csrc/common.h",
                  "gemm_epilogue_fuse_amd/csrc/kernel_decode.h", "gemm_epilogue_fuse_amd/csrc/kernel_strip.h",
                  "gemm_epilogue_fuse_amd/csrc/launch.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- timing

# Untimed launches before the warmup steps, long enough for the GPU clocks to
# leave their idle state (a few ms of launches after an idle host phase
# measured about 10% slow).
SETTLE_S = 0.3


def time_calls(fn_for_set, nsets, steps, warmup, settle_s=None):
    """Run fn_for_set(i % nsets) for settle_s seconds, then warmup + steps
    times.  Returns (wall ms/step, device ms per launch): HIP events on the
    launching stream bracket the whole batch of back-to-back launches, so
    short kernels are not charged for the host's gap between calls."""
    import torch
    t_end = time.perf_counter() + (SETTLE_S if settle_s is None else settle_s)
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(16):
            fn_for_set(i % nsets)
            i += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        fn_for_set(i % nsets)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fn_for_set(i % nsets)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    dev_ms = e0.elapsed_time(e1) / steps
    return wall_ms, dev_ms


def launch_floor_us(steps=200, graph=False):
    """Device time per launch of a one-element device op, timed like the
    kernels (eager, or by HIP-graph replay): the floor under any call's
    latency."""
    import torch
    x = torch.zeros(1, device="cuda:0")
    if graph:
        return round(graph_time_ms(lambda i, strm: x.add_(1.0), 1) * 1e3, 3)
    _, dev = time_calls(lambda i: x.add_(1.0), 1, steps, 20)
    return round(dev * 1e3, 3)


def rotating_sets(make, bytes_per_set):
    n = max(2, min(64, (ROTATE_BYTES + bytes_per_set - 1) // bytes_per_set))
    return [make(i) for i in range(n)]


# ----------------------------------------------------------------------------- workloads

def rms_linear_sets(M, D, N, dtype_s, seed=0, order=("X", "gamma", "W")):
    import synth
    d = synth.rmsnorm_linear(M=M, D=D, N=N, seed=seed, dtype=dtype_s, order=order,
                             w_std=1.0 / (D ** 0.5))
    base = {k: synth.to_torch(v, dtype_s, "cuda:0") for k, v in d.items()}
    per_set = (M * D + D + D * N + M * N) * 2

    def make(i):
        if i == 0:
            t = dict(base)
        else:
            t = {k: v.clone() for k, v in base.items()}
        t["Y"] = torch_empty((M, N), base["X"].dtype)
        return t
    return d, rotating_sets(make, per_set)


def torch_empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="cuda:0")


def bench_rms_linear(M, D, N, dtype_s, steps, warmup, order=("X", "gamma", "W"), graph=False):
    """Time fuse_rmsnorm_gemm through the C ABI with pre-marshalled pointers
    (what a native caller does), so host-side Python cost stays out of the way."""
    import ctypes
    import torch
    import gemm_epilogue_fuse_amd as lf
    d, sets = rms_linear_sets(M, D, N, dtype_s, order=order)
    L = lf.lib()
    code = lf.BF16 if dtype_s == "bf16" else lf.F16
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    eps = ctypes.c_float(EPS)
    argv = [(s["X"].data_ptr(), s["gamma"].data_ptr(), s["W"].data_ptr(), s["Y"].data_ptr()) for s in sets]
    fn = L.fuse_rmsnorm_gemm

    def call_on(i, strm):
        x, g, w, y = argv[i]
        rc = fn(x, g, eps, w, None, y, M, N, D, 0, code, strm)
        if rc:
            raise lf.FuseError(rc, "fuse_rmsnorm_gemm")

    def call(i):
        call_on(i, stream)
    wall, dev = time_calls(call, len(sets), steps, warmup)
    flops = 2.0 * M * N * D
    alg_bytes = (M * D + D + D * N + M * N) * 2
    if graph:
        gdev = graph_time_ms(call_on, len(sets))
        return d, sets, wall, dev, flops, alg_bytes, gdev
    return d, sets, wall, dev, flops, alg_bytes


def graph_time_ms(call_on, nsets, launches=40, replays=10):
    """Device ms per launch from a HIP graph of `launches` back-to-back calls
    over the rotating input sets, replayed `replays` times: no host launch
    gap between kernels, so short calls show their device time."""
    import ctypes
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    sp = ctypes.c_void_p(s.cuda_stream)
    with torch.cuda.stream(s):
        for i in range(nsets):  # per-stream library state (split-K workspace) exists before capture
            call_on(i, sp)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(launches):
            call_on(i % nsets, sp)
    with torch.cuda.stream(s):
        for _ in range(3):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
    s.synchronize()
    return e0.elapsed_time(e1) / (launches * replays)


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
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    or None if absent or taken on a different kernel source."""
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
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(min_seconds=10.0):
    """The fp64 oracle, as it stands, on the same workload (whole 512x4096x4096
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


# ----------------------------------------------------------------------------- sweep

def sweep(steps, warmup, only=None):
    """One JSON line per workload on stderr; `only` keeps the workloads whose
    name contains it (for profiling one kernel at a time)."""
    import torch
    import gemm_epilogue_fuse_amd as lf
    import synth

    def emit(rec):
        print(json.dumps(rec), file=sys.stderr, flush=True)

    def want(name):
        return only is None or only in name

    # GEMM + bias + activation, N = K = 4096
    for M, act, resid in [(512, "gelu_tanh", False), (1024, "gelu_tanh", False), (2048, "gelu_tanh", False),
                          (4096, "gelu_tanh", False), (4096, "silu", False), (4096, "relu", False),
                          (4096, "none", True)]:
        N = K = 4096
        name = "gemm_bias_%s%s_%dx4096x4096_fp16" % (act, "_residual" if resid else "", M)
        if not want(name):
            continue
        d = synth.gemm_epilogue_sweep(M, N, K, seed=0, residual=resid)
        base = {k: synth.to_torch(v, synth.F16, "cuda:0") for k, v in d.items()}
        per = (M * K + K * N + N + M * N * (2 if resid else 1)) * 2

        def make(i, base=base, M=M, N=N):
            t = base if i == 0 else {k: v.clone() for k, v in base.items()}
            t = dict(t)
            t["Y"] = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
            return t
        sets = rotating_sets(make, per)

        def call(i, sets=sets, act=act):
            s = sets[i]
            lf.gemm_epilogue(s["A"], s["W"], s["bias"], s.get("R"), act, out=s["Y"])
        _, dev = time_calls(call, len(sets), steps, warmup)
        rec = {"workload": name, "plan": lf.plan_name(0, M, N, K)}
        rec.update(result_fields(dev, 2.0 * M * N * K, per))
        emit(rec)
        del sets, base

    # The same work unfused through the vendor library, for context: torch's
    # rms_norm, matmul (hipBLASLt) and elementwise kernels, timed the same way
    # (warm inputs: one set).
    def unfused(name, fn, flops, alg):
        if not want(name):
            return
        _, dev = time_calls(lambda i: fn(), 1, steps, warmup)
        rec = {"workload": name, "plan": "torch (hipBLASLt matmul + separate elementwise kernels)"}
        rec.update(result_fields(dev, flops, alg))
        emit(rec)

    F = torch.nn.functional
    X = torch.randn(512, 4096, device="cuda:0").half()
    g = (1 + 0.1 * torch.randn(4096, device="cuda:0")).half()
    W = (torch.randn(4096, 4096, device="cuda:0") / 64).half()
    unfused("unfused_rmsnorm_then_matmul_512x4096x4096_fp16",
            lambda: torch.matmul(F.rms_norm(X, (4096,), g, EPS), W),
            2.0 * 512 * 4096 * 4096, (2 * 512 * 4096 + 4096 + 4096 * 4096) * 2)
    A = torch.randn(4096, 4096, device="cuda:0").half()
    bias = (0.1 * torch.randn(4096, device="cuda:0")).half()
    unfused("unfused_matmul_bias_gelu_tanh_4096x4096x4096_fp16",
            lambda: F.gelu(torch.matmul(A, W) + bias, approximate="tanh"),
            2.0 * 4096 ** 3, (3 * 4096 * 4096 + 4096) * 2)
    del X, g, W, A, bias

    # SwiGLU FFN block, bf16: kernel 1 (RMSNorm + gate/up + SiLU*up), kernel 2 (down + bias + residual)
    M, D, F = 2048, 4096, 11008
    n1 = "swiglu_k1_rmsnorm_gate_up_2048x11008x4096_bf16"
    n2 = "swiglu_k2_down_bias_residual_2048x4096x11008_bf16"
    n3 = "swiglu_ffn_block_bf16_total"
    if want(n1) or want(n2) or want(n3):
        swiglu_block(lf, synth, emit, steps, warmup, M, D, F, n1, n2, n3)

    # decode-shaped RMSNorm -> Linear, timed by HIP-graph replay (eager
    # launches of a few-microsecond kernel measure the host's launch rate);
    # cells whose roofline time is under the launch floor cannot show their
    # HBM fraction and are flagged
    floor = launch_floor_us(graph=True)
    if want("launch_floor_one_element_op"):
        emit({"workload": "launch_floor_one_element_op", "latency_us": floor,
              "timing": "HIP graph of 40 launches, replayed", "eager_latency_us": launch_floor_us()})
    for dt in (synth.F16, synth.BF16):
        for D in (1024, 2048, 4096):
            for B in (1, 32, 128, 512, 1024):
                name = "decode_rmsnorm_linear_B%d_D%d_%s" % (B, D, dt)
                if not want(name):
                    continue
                _, sets, _, dev, flops, alg, gdev = bench_rms_linear(B, D, D, dt, steps, warmup,
                                                                     order=("W", "X", "gamma"), graph=True)
                rec = {"workload": name,
                       "plan": lf.plan_name(1, B, D, D, lf.BF16 if dt == synth.BF16 else lf.F16),
                       "timing": "HIP graph of 40 launches, replayed"}
                rec.update(result_fields(gdev, flops, alg))
                rec["eager_latency_us"] = round(dev * 1e3, 3)
                rec["launch_floor_us"] = floor
                rec["below_launch_floor"] = rec["roof_us"] < floor
                emit(rec)
                del sets


def swiglu_block(lf, synth, emit, steps, warmup, M, D, F, n1, n2, n3):
    """SwiGLU FFN block in bf16: kernel 1 (RMSNorm + gate/up + SiLU*up) and
    kernel 2 (down + bias + residual)."""
    import torch
    d = synth.swiglu_ffn(M=M, D=D, F=F, seed=0)
    t = {k: synth.to_torch(v, synth.BF16, "cuda:0") for k, v in d.items()}
    H = torch.empty((M, F), dtype=torch.bfloat16, device="cuda:0")
    Y = torch.empty((M, D), dtype=torch.bfloat16, device="cuda:0")
    _, dev1 = time_calls(lambda i: lf.rmsnorm_gemm_swiglu(t["X"], t["gamma"], t["Wg"], t["Wu"], EPS, out=H),
                         1, steps, warmup)
    _, dev2 = time_calls(lambda i: lf.gemm_epilogue(H, t["Wd"], t["bias"], t["X"], "none", out=Y), 1, steps, warmup)
    b1 = (M * D + D + 2 * D * F + M * F) * 2
    b2 = (M * F + F * D + D + 2 * M * D) * 2
    r1 = {"workload": n1, "plan": lf.plan_name(2, M, F, D, lf.BF16)}
    r1.update(result_fields(dev1, 4.0 * M * F * D, b1))
    emit(r1)
    r2 = {"workload": n2, "plan": lf.plan_name(0, M, D, F, lf.BF16)}
    r2.update(result_fields(dev2, 2.0 * M * D * F, b2))
    emit(r2)
    r3 = {"workload": n3}
    r3.update(result_fields(dev1 + dev2, 4.0 * M * F * D + 2.0 * M * D * F, b1 + b2))
    emit(r3)


# ----------------------------------------------------------------------------- main

def main():
    global SETTLE_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--only", default=None, help="with --sweep: only the workloads whose name contains this")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed launches before the warmup steps (0 under counter runs)")
    args = ap.parse_args()
    SETTLE_S = max(0.0, args.settle)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build runs the fused kernels on a single MI355X "
              "(no multi-GPU path); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_epilogue_fuse_amd as lf
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

    M, D, N = 512, 4096, 4096
    d, sets, wall_ms, dev_ms, flops, alg = bench_rms_linear(M, D, N, "f16", args.steps, args.warmup)
    fields = result_fields(dev_ms, flops, alg)
    value = flops / (wall_ms * 1e-3) / 1e12       # whole-job throughput over the timed region
    plan = lf.plan_name(1, M, N, D)
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
        "config": {"workload": "rmsnorm_linear_512x4096x4096_fp16", "M": M, "K": D, "N": N, "eps": EPS,
                   "bias": None, "act": "none", "seed": 0, "plan": plan, "rotating_input_sets": len(sets),
                   "clock_settle_s": SETTLE_S, "parallelism": "none (1 GPU)"},
        "latency_us": fields["latency_us"],
        "hbm_gbs": fields["hbm_gbs"],
        "mfma_frac": fields["mfma_frac"],
        "hbm_frac": fields["hbm_frac"],
        "roofline": {"bound": "mfma", "achieved": fields["tflops"], "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": fields["mfma_frac"], "traffic": traffic,
                     "algorithmic_bytes": alg, "kernel": "%s (plan %s)" % ("gemm_dma_kernel" if plan.startswith("dma") else "gemm_fused_kernel", plan),
                     "kernel_source_sha256_16": kernel_hash()},
        "baseline_context": "0.208 ms fused on an NVIDIA A30 (page figure, other hardware); vs_baseline = 0.208 ms / ms_per_step",
    }
    del sets
    if not args.no_cpu:
        log("timing the fp64 oracle on the host cores ...")
        rec["cpu_baseline"] = cpu_baseline()
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    if args.sweep:
        sweep(max(20, args.steps // 4), max(5, args.warmup // 2), args.only)


if __name__ == "__main__":
    main()
