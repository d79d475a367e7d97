"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the roofline
fields and the rule that stored traffic counters apply only to the kernel
sources they were taken on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_result_fields_roofline():
    # 512x4096x4096 RMSNorm -> Linear: 17.18 GFLOP, 41.95 MB algorithmic
    flops = 2.0 * 512 * 4096 * 4096
    alg = (512 * 4096 + 4096 + 4096 * 4096 + 512 * 4096) * 2
    f = bench.result_fields(0.0312, flops, alg)  # 31.2 us per launch
    assert f["latency_us"] == pytest.approx(31.2)
    assert f["tflops"] == pytest.approx(flops / 31.2e-6 / 1e12, rel=1e-3)
    assert f["mfma_frac"] == pytest.approx(f["tflops"] / bench.PEAK_MFMA_TFLOPS, rel=1e-3)
    assert f["hbm_frac"] == pytest.approx(alg / 31.2e-6 / 1e9 / bench.PEAK_HBM_GBS, rel=1e-3)
    # arithmetic intensity 409.6 flop/B is above the 312.5 ridge: matrix-core bound
    assert f["roof_bound"] == "mfma"
    assert f["roof_us"] == pytest.approx(flops / (bench.PEAK_MFMA_TFLOPS * 1e12) * 1e6, rel=1e-3)
    # a decode-shaped call (B=1, D=4096) is bound by HBM
    g = bench.result_fields(0.0137, 2.0 * 4096 * 4096, (2 * 4096 + 4096 + 4096 * 4096) * 2)
    assert g["roof_bound"] == "hbm"


def test_traffic_counters_follow_the_kernel_sources(monkeypatch):
    name = "rmsnorm_linear_512x4096x4096_fp16.traffic.txt"
    if not os.path.exists(os.path.join(ROOT, "profiles", name)):
        pytest.skip("no stored traffic summary")
    with open(os.path.join(ROOT, "profiles", name)) as f:
        stored = [ln.split(":", 1)[1].strip() for ln in f if ln.startswith("kernel_source_sha256_16:")][0]
    monkeypatch.setattr(bench, "kernel_hash", lambda: stored)
    assert bench.read_traffic(name) > 0
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.read_traffic(name) is None
    assert bench.read_traffic("no_such_summary.txt") is None


def test_kernel_sources_cover_every_device_source():
    """The counter-validity hash covers every file compiled into libfuse's kernels."""
    csrc = os.path.join(ROOT, "gemm_epilogue_fuse_amd", "csrc")
    device = sorted("gemm_epilogue_fuse_amd/csrc/" + f for f in os.listdir(csrc) if f.endswith((".h", ".hip")))
    assert sorted(bench.KERNEL_SOURCES) == device


def test_workload_list_covers_every_config():
    """The default run times every workload of the operator's configuration list."""
    import gemm_epilogue_fuse_amd as lf
    names = [w.name for w in bench.all_workloads(lf)]
    assert "gemm_bias_gelu_tanh_64x256x256_fp16" in names
    for M in (512, 1024, 2048, 4096):
        assert "gemm_bias_gelu_tanh_%dx4096x4096_fp16" % M in names
    for v in ("silu", "relu", "residual"):
        assert "gemm_bias_%s_4096x4096x4096_fp16" % v in names
    assert sum(n.startswith("swiglu_") for n in names) == 3
    dec = [n for n in names if n.startswith("decode_rmsnorm_linear_")]
    assert len(dec) == 30 and len(set(dec)) == 30
