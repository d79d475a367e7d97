"""Graph-level fusion on the device (needs an MI355X): each model rewritten by
gemm_epilogue_fuse_amd.fx runs its fused libfuse calls and matches the same
model evaluated unfused by torch in float32 (with the same fp16 weights and
inputs), within max_abs_err <= 1.5e-2 and mean_abs_err <= 1.5e-3."""
import numpy as np
import pytest
import torch

from gemm_epilogue_fuse_amd import fx as lfx
import fx_models as M
from parity_util import assert_close, say

pytestmark = pytest.mark.gpu

CASES = [
    ("rms_linear_gelu", lambda: M.RmsLinearGelu(512, 264), [(4, 37, 512)], ["rmsnorm_gemm"]),
    ("decomposed_rms_q", lambda: M.DecomposedRmsQProj(512, 512), [(130, 512)], ["rmsnorm_gemm"]),
    ("shared_norm_qkv", lambda: M.SharedNormQKV(256), [(64, 256)], ["gemm_epilogue"] * 3),
    ("swiglu_mlp", lambda: M.SwiGluMlp(512, 1376), [(2, 100, 512)], ["rmsnorm_swiglu", "gemm_epilogue"]),
    ("ln_linear_relu", lambda: M.LnLinearRelu(384, 200), [(300, 384)], ["layernorm_gemm"]),
    ("prologue_bias", lambda: M.PrologueBias(64, 16), [(16, 64)], ["prologue_bias_gemm"]),
    ("matmul_bias_act_residual", lambda: M.MatmulBiasActResidual(256, 136), [(96, 256), (96, 136)],
     ["gemm_epilogue", "gemm_epilogue"]),
]


def randomise_norms(model, g):
    for mod in model.modules():
        if isinstance(mod, (torch.nn.RMSNorm, torch.nn.LayerNorm, M.DecomposedRmsNorm)):
            with torch.no_grad():
                mod.weight.copy_(1.0 + 0.1 * torch.randn(mod.weight.shape, generator=g))
                if getattr(mod, "bias", None) is not None and isinstance(mod.bias, torch.nn.Parameter):
                    mod.bias.copy_(0.1 * torch.randn(mod.bias.shape, generator=g))


@pytest.mark.parametrize("name,make,shapes,patterns", CASES, ids=[c[0] for c in CASES])
def test_fused_graph_matches_unfused_model(name, make, shapes, patterns):
    g = torch.Generator().manual_seed(7)
    model = make()
    randomise_norms(model, g)
    model = model.half().cuda().eval()
    inputs = [torch.randn(s, generator=g).half().cuda() for s in shapes]
    say("fx", name, shapes)
    gm, applied = lfx.fuse_graph(model, *inputs)
    assert sorted(applied) == sorted(patterns)
    with torch.no_grad():
        got = gm(*inputs)
        ref = model.float()(*[x.float() for x in inputs])
    got = got if isinstance(got, tuple) else (got,)
    ref = ref if isinstance(ref, tuple) else (ref,)
    for a, b in zip(got, ref):
        assert a.dtype == torch.float16 and a.shape == b.shape
        assert_close(a.double().cpu().numpy(), b.double().cpu().numpy(), name)
