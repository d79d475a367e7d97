"""Auto-tuner for libfuse's tile plans, with a persistent JSON cache.

"llm-fusion-compiler", Auto-Tuner: a grid search over tile configurations
under the hardware's limits, each candidate timed on the device, the winner
kept in a persistent JSON cache per (pattern, shape, architecture), and a
heuristic fallback where no device can time them.  Here:

* the search space is every compiled plan that can serve the call
  (``fuse_plan_applies``), crossed with K-split counts for the plans that
  split K;
* the hardware limits of gfx950 (at most 160 KiB of LDS per workgroup, at
  most 1024 threads, whole 64-wide waves) and the 64 MiB split-K workspace
  are checked against what the HIP runtime reports for each candidate's
  kernel (``fuse_kernel_resources``) and ``fuse_workspace_bytes``;
* each candidate is timed as a HIP graph of back-to-back calls, over enough
  input sets that consecutive calls miss the last-level cache;
* the cache maps "op|M|N|K|dtype|arch" to the winning plan (with its time,
  the static choice's time and every candidate's), and ``load_cache``
  registers the entries of the running architecture with
  ``fuse_tune_set``, which the library consults before its static rules;
* without a GPU, ``tune`` returns the library's static choice (the
  heuristic) and writes nothing.

Setting LIBFUSE_TUNE_CACHE to a cache file makes ``gemm_epilogue_fuse_amd``
load it when the library is first used.

    python -m gemm_epilogue_fuse_amd.tuner --op rmsnorm_gemm --shape 512 4096 4096 --dtype f16
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import time

from . import BF16, F16, FuseError, lib, plan_name, workspace_bytes

ARCH = "gfx950"
LDS_LIMIT = 160 * 1024     # bytes of LDS a workgroup may hold on gfx950
THREADS_LIMIT = 1024       # threads per workgroup
WAVE = 64
WORKSPACE_LIMIT = 64 << 20  # the first split-K buffer of a stream
SPLITS = (1, 2, 3, 4, 6, 8, 12, 16)
OPS = {"gemm_epilogue": 0, "rmsnorm_gemm": 1, "rmsnorm_gemm_swiglu": 2, "layernorm_gemm": 3,
       "gemm_prologue_bias": 4}
OP_NAMES = {v: k for k, v in OPS.items()}
DTYPES = {"f16": F16, "bf16": BF16}


def cache_path() -> str:
    return os.environ.get("LIBFUSE_TUNE_CACHE") or os.path.join(os.path.expanduser("~"), ".cache", "libfuse",
                                                                 "tune_%s.json" % ARCH)


def cache_key(op: int, M: int, N: int, K: int, dtype: int, arch: str = ARCH) -> str:
    return "%s|%d|%d|%d|%s|%s" % (OP_NAMES[op], M, N, K, "bf16" if (dtype & 0xff) == BF16 else "f16", arch)


def parse_key(key: str):
    op, M, N, K, dt, arch = key.split("|")
    return OPS[op], int(M), int(N), int(K), DTYPES[dt], arch


def read_cache(path: str | None = None) -> dict:
    path = path or cache_path()
    if not os.path.exists(path):
        return {"version": 1, "entries": {}}
    with open(path) as f:
        data = json.load(f)
    if data.get("version") != 1 or not isinstance(data.get("entries"), dict):
        raise ValueError("%s is not a libfuse tune cache (version 1)" % path)
    return data


def write_cache(data: dict, path: str | None = None) -> str:
    path = path or cache_path()
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    tmp = path + ".tmp%d" % os.getpid()
    with open(tmp, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    os.replace(tmp, path)
    return path


def set_tuned(op: int, M: int, N: int, K: int, dtype: int, plan: str | None) -> None:
    rc = lib().fuse_tune_set(op, M, N, K, dtype, None if plan is None else plan.encode())
    if rc != 0:
        raise FuseError(rc, "fuse_tune_set")


def load_cache(path: str | None = None, arch: str = ARCH) -> int:
    """Register every entry of the cache for `arch` with the library; returns
    how many were registered (entries whose plan no longer fits are skipped)."""
    n = 0
    for key, ent in read_cache(path)["entries"].items():
        op, M, N, K, dt, a = parse_key(key)
        if a != arch:
            continue
        if lib().fuse_tune_set(op, M, N, K, dt, ent["plan"].encode()) == 0:
            n += 1
    return n


def plans():
    """The compiled plans: (name, fields) with fields = BM, BN, BK, stages,
    threads, can split K, dual GEMM, kernel family."""
    L = lib()
    out = []
    f = (ctypes.c_int32 * 8)()
    for i in range(L.fuse_plan_count()):
        name = L.fuse_plan_info(i, f)
        out.append((name.decode(), list(f)))
    return out


def candidates(op: int, M: int, N: int, K: int, dtype: int = F16):
    """Plan strings that can serve the call: every fitting plan, and for plans
    that split K every split count in SPLITS that leaves each split at least
    two K steps (counts that clamp to the same split are listed once)."""
    L = lib()
    out = []
    for name, f in plans():
        if not L.fuse_plan_applies(op, M, N, K, dtype, name.encode()):
            continue
        bk, can_split = f[2], f[5]
        nk = K // bk
        seen = set()
        for s in (SPLITS if can_split else (1,)):
            if s > 1 and nk // s < 2:
                break
            label = name if s == 1 else "%s:k%d" % (name, s)
            set_tuned(op, M, N, K, dtype, label)
            eff = plan_name(op, M, N, K, dtype)  # what the library runs for it
            set_tuned(op, M, N, K, dtype, None)
            if eff in seen:
                continue
            seen.add(eff)
            out.append(eff)
    return out


def within_limits(res) -> bool:
    """res = (LDS bytes, launch threads, max threads per block, registers, scratch)."""
    lds, threads, max_threads = res[0], res[1], res[2]
    return lds <= LDS_LIMIT and threads <= THREADS_LIMIT and threads <= max_threads and threads % WAVE == 0


def resources(op: int, M: int, N: int, K: int, dtype: int):
    out = (ctypes.c_int32 * 5)()
    rc = lib().fuse_kernel_resources(op, M, N, K, dtype, out)
    if rc != 0:
        raise FuseError(rc, "fuse_kernel_resources")
    return list(out)


def heuristic(op: int, M: int, N: int, K: int, dtype: int = F16) -> str:
    """The library's static shape rules (what runs without a tuned entry)."""
    set_tuned(op, M, N, K, dtype, None)
    return plan_name(op, M, N, K, dtype)


# ----------------------------------------------------------------------------- timing on the device

ROTATE_BYTES = 640 << 20  # input footprint of a timing: past the 256 MB last-level cache


def _set_bytes(op, M, N, K):
    return 2 * (M * K + K * N * (2 if op == 2 else 1) + M * N + 2 * K + N)


def _inputs(op, M, N, K, dtype, nsets=2):
    import torch
    tdt = torch.bfloat16 if (dtype & 0xff) == BF16 else torch.float16
    g = torch.Generator(device="cuda").manual_seed(0)

    def r(*shape, std=1.0, mean=0.0):
        return (torch.randn(*shape, generator=g, device="cuda") * std + mean).to(tdt)
    sets = []
    for _ in range(nsets):
        s = {"A": r(M, K), "W": r(K, N, std=K ** -0.5), "bias": r(N, std=0.1), "Y": torch.empty(M, N, dtype=tdt,
                                                                                                device="cuda")}
        if op in (1, 2, 3):
            s["gamma"] = r(K, std=0.1, mean=1.0)
        if op == 2:
            s["W2"] = r(K, N, std=K ** -0.5)
        if op == 3:
            s["beta"] = r(K, std=0.1)
        if op == 4:
            s["abias"] = r(K, std=0.1)
        sets.append(s)
    return sets


def _caller(op, M, N, K, dtype, s):
    L = lib()
    eps = ctypes.c_float(1e-6)
    p = {k: v.data_ptr() for k, v in s.items()}
    if op == 0:
        return lambda st: L.fuse_gemm_epilogue(p["A"], p["W"], p["bias"], None, p["Y"], M, N, K, 0, dtype, st)
    if op == 1:
        return lambda st: L.fuse_rmsnorm_gemm(p["A"], p["gamma"], eps, p["W"], None, p["Y"], M, N, K, 0, dtype, st)
    if op == 2:
        return lambda st: L.fuse_rmsnorm_gemm_swiglu(p["A"], p["gamma"], eps, p["W"], p["W2"], p["Y"], M, N, K,
                                                     dtype, st)
    if op == 3:
        return lambda st: L.fuse_layernorm_gemm(p["A"], p["gamma"], p["beta"], eps, p["W"], p["bias"], p["Y"], M,
                                                N, K, 0, dtype, st)
    return lambda st: L.fuse_gemm_prologue_bias(p["A"], p["abias"], p["W"], p["bias"], None, p["Y"], M, N, K, 0,
                                                dtype, st)


def _time_us(calls, launches, replays=3):
    """Device microseconds per call: a HIP graph of `launches` calls over the
    input sets, after eager calls that create any per-stream state."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    st = ctypes.c_void_p(s.cuda_stream)
    with torch.cuda.stream(s):
        for c in calls * 3:
            rc = c(st)
            if rc:
                raise FuseError(rc, "libfuse call")
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(launches):
            calls[i % len(calls)](st)
    with torch.cuda.stream(s):
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(replays):
            g.replay()
        e1.record(s)
    s.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (launches * replays)


def tune(op: int, M: int, N: int, K: int, dtype: int = F16, launches: int = 20, path: str | None = None,
         write: bool = True, max_candidates: int | None = None, cold: bool = True) -> dict:
    """Time every candidate plan for the call, register the fastest and (with
    `write`) store it in the cache.  `cold` rotates over enough input sets that
    consecutive calls miss the last-level cache (a model's layer after layer);
    otherwise two sets.  Without a GPU: the heuristic choice."""
    import torch
    if not torch.cuda.is_available():
        return {"plan": heuristic(op, M, N, K, dtype), "source": "heuristic"}
    default = heuristic(op, M, N, K, dtype)
    cands = candidates(op, M, N, K, dtype)
    if max_candidates is not None:
        cands = ([default] + [c for c in cands if c != default])[:max_candidates]
    nsets = max(2, min(64, -(-ROTATE_BYTES // _set_bytes(op, M, N, K)))) if cold else 2
    sets = _inputs(op, M, N, K, dtype, nsets)
    launches = max(launches, nsets)
    times = {}
    try:
        for c in cands:
            set_tuned(op, M, N, K, dtype, c)
            if workspace_bytes(op, M, N, K, dtype) > WORKSPACE_LIMIT:
                continue
            if not within_limits(resources(op, M, N, K, dtype)):
                continue
            calls = [_caller(op, M, N, K, dtype, s) for s in sets]
            times[c] = _time_us(calls, launches)
    finally:
        set_tuned(op, M, N, K, dtype, None)
    best = min(times, key=times.get)
    set_tuned(op, M, N, K, dtype, best)
    ent = {"plan": best, "us": round(times[best], 3), "default_plan": default, "cold": cold,
           "default_us": round(times[default], 3) if default in times else None,
           "candidates": {k: round(v, 3) for k, v in sorted(times.items(), key=lambda kv: kv[1])},
           "tuned_at": time.strftime("%Y-%m-%dT%H:%M:%S")}
    if write:
        data = read_cache(path)
        data["entries"][cache_key(op, M, N, K, dtype)] = ent
        write_cache(data, path)
    return dict(ent, source="measured")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--op", choices=sorted(OPS), required=True)
    ap.add_argument("--shape", type=int, nargs=3, metavar=("M", "N", "K"), required=True)
    ap.add_argument("--dtype", choices=sorted(DTYPES), default="f16")
    ap.add_argument("--cache", default=None, help="cache file (default: %s)" % cache_path())
    ap.add_argument("--launches", type=int, default=20)
    args = ap.parse_args()
    M, N, K = args.shape
    print(json.dumps(tune(OPS[args.op], M, N, K, DTYPES[args.dtype], args.launches, args.cache)))


if __name__ == "__main__":
    main()
