"""The tuner's host logic (no GPU): plan enumeration, the candidate space
under each op's constraints, the hardware-limit filter, the tuned-plan table
of the library and the persistent JSON cache ("llm-fusion-compiler",
Auto-Tuner: search space, constraints, cache, heuristic fallback)."""
import json
import os
import subprocess
import sys

import pytest

import gemm_epilogue_fuse_amd as lf
from gemm_epilogue_fuse_amd import tuner

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(autouse=True)
def clean_table():
    lf.set_plan(None)
    lf.lib().fuse_tune_clear()
    yield
    lf.lib().fuse_tune_clear()


def test_plans_are_enumerated_with_their_shapes():
    ps = tuner.plans()
    names = [n for n, _ in ps]
    assert len(names) == len(set(names)) == lf.lib().fuse_plan_count()
    assert "dma_128x128x64_s4_g2" in names and "dec_32x64" in names and "reg_256x256x64" in names
    for name, f in ps:
        bm, bn, bk, stages, threads, can_split, dual, kind = f
        assert bm > 0 and bn > 0 and bk > 0 and threads % 64 == 0 and threads <= 1024, name
        assert str(bm) in name and str(bn) in name
        assert dual == ("dual" in name)
    assert lf.lib().fuse_plan_info(len(ps), (tuner.ctypes.c_int32 * 8)()) is None


def test_candidates_follow_each_ops_constraints():
    # K not a multiple of 64: only the register-staged plans
    c = tuner.candidates(0, 300, 392, 328)
    assert c and all(x.startswith("reg_") for x in c)
    # a decode shape: few-row kernels and split counts, every label once
    c = tuner.candidates(1, 1, 1024, 1024)
    assert "wstrip_16x16" in c and "strip_16x16" in c and any(x.startswith("dec_32x64") for x in c)
    assert len(c) == len(set(c))
    # split labels clamp like the library: the small-M kernel needs chunks of at most 8 steps
    c = tuner.candidates(1, 32, 4096, 4096)
    assert "dec_32x64:k8" in c and "dec_32x64:k2" not in c
    # the gate/up pair only has the dual plans; LayerNorm and the input bias the register-staged
    # plans and the 4 x 1 wave LDS-DMA tiles
    assert all("dual" in x for x in tuner.candidates(2, 512, 1024, 1024))
    ln_tiles = ("dma_256x256x32_s4", "dma_256x128x64_s3", "dma_128x128x64_s4")
    bias_tiles = ln_tiles + ("dma_256x256x32_s4_w8", "dma_256x128x64_s3_w8")
    for op, tiles in ((3, ln_tiles), (4, bias_tiles)):
        c = tuner.candidates(op, 512, 1024, 1024)
        assert all(x.split(":")[0] in tiles or x.startswith("reg_") for x in c), c
        assert all(any(x.split(":")[0] == t for x in c) for t in tiles) and any(x.startswith("reg_") for x in c), c
    # enumerating candidates leaves no entry behind
    assert lf.plan_name(1, 32, 4096, 4096) == tuner.heuristic(1, 32, 4096, 4096)


def test_hardware_limit_filter():
    assert tuner.within_limits([135936, 512, 512, 222, 0])
    assert not tuner.within_limits([170000, 256, 256, 128, 0])    # over 160 KiB of LDS
    assert not tuner.within_limits([65536, 2048, 2048, 64, 0])    # over 1024 threads
    assert not tuner.within_limits([65536, 512, 256, 64, 0])      # launch bounds smaller than the launch
    assert not tuner.within_limits([65536, 96, 96, 64, 0])        # not whole waves


def test_tuned_table_is_consulted_before_the_static_rules():
    assert lf.plan_name(0, 512, 4096, 4096) == "dma_128x128x64_s4_g2:k2"
    tuner.set_tuned(0, 512, 4096, 4096, lf.F16, "dma_256x128x64_s3_w8:k4")
    assert lf.plan_name(0, 512, 4096, 4096) == "dma_256x128x64_s3_w8:k4"
    # exact keys: other shapes, ops and dtypes keep the static rules
    assert lf.plan_name(0, 512, 4096, 2048) != "dma_256x128x64_s3_w8:k4"
    assert lf.plan_name(1, 512, 4096, 4096) == "dma_128x128x64_s4_g2:k2"
    assert lf.plan_name(0, 512, 4096, 4096, lf.BF16) == "dma_128x128x64_s4_g2:k2"
    # a forced plan still wins over the table
    lf.set_plan("dma_128x128x64_s4")
    assert lf.plan_name(0, 512, 4096, 4096) == "dma_128x128x64_s4"
    lf.set_plan(None)
    # plans that cannot serve the call, and unknown names, are refused
    with pytest.raises(lf.FuseError):
        tuner.set_tuned(0, 512, 4096, 4096, lf.F16, "dma_dual_256x128x32_s4")
    with pytest.raises(lf.FuseError):
        tuner.set_tuned(0, 300, 392, 328, lf.F16, "dma_128x128x64_s4")  # K % 64 != 0
    with pytest.raises(lf.FuseError):
        tuner.set_tuned(0, 512, 4096, 4096, lf.F16, "no_such_plan")
    tuner.set_tuned(0, 512, 4096, 4096, lf.F16, None)
    assert lf.plan_name(0, 512, 4096, 4096) == "dma_128x128x64_s4_g2:k2"


def test_cache_round_trip(tmp_path):
    path = str(tmp_path / "tune.json")
    data = {"version": 1, "entries": {
        tuner.cache_key(1, 512, 4096, 4096, lf.F16): {"plan": "dma_64x128x64_s4_g2:k3", "us": 1.0},
        tuner.cache_key(0, 4096, 4096, 4096, lf.F16, arch="gfx942"): {"plan": "dma_128x128x64_s4", "us": 1.0},
        tuner.cache_key(0, 300, 392, 328, lf.BF16): {"plan": "dma_128x128x64_s4", "us": 1.0},  # no longer fits
    }}
    tuner.write_cache(data, path)
    assert tuner.read_cache(path) == data
    assert tuner.load_cache(path) == 1  # only this architecture's entries that still fit
    assert lf.plan_name(1, 512, 4096, 4096) == "dma_64x128x64_s4_g2:k3"
    assert lf.plan_name(0, 4096, 4096, 4096) == "dma_256x256x32_s4_w8"
    assert tuner.parse_key(tuner.cache_key(2, 2048, 11008, 4096, lf.BF16)) == (2, 2048, 11008, 4096, lf.BF16,
                                                                               "gfx950")
    with open(path, "w") as f:
        json.dump({"version": 7}, f)
    with pytest.raises(ValueError):
        tuner.read_cache(path)
    assert tuner.read_cache(str(tmp_path / "missing.json")) == {"version": 1, "entries": {}}


def test_cache_named_by_the_environment_is_loaded_with_the_library(tmp_path):
    path = str(tmp_path / "tune.json")
    tuner.write_cache({"version": 1, "entries": {
        tuner.cache_key(0, 1024, 4096, 4096, lf.F16): {"plan": "dma_256x128x64_s3_w8", "us": 1.0}}}, path)
    code = ("import gemm_epilogue_fuse_amd as lf; print(lf.plan_name(0, 1024, 4096, 4096))")
    env = dict(os.environ, LIBFUSE_TUNE_CACHE=path, PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=120)
    assert out.stdout.strip() == "dma_256x128x64_s3_w8", out.stderr
    env.pop("LIBFUSE_TUNE_CACHE")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=120)
    assert out.stdout.strip() == "dma_128x128x64_s4_g2"


def test_heuristic_fallback_without_a_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: tune() measures instead")
    r = tuner.tune(1, 512, 4096, 4096, write=False)
    assert r == {"plan": "dma_128x128x64_s4_g2:k2", "source": "heuristic"}
