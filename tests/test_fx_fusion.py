"""Graph-level fusion on torch.fx graphs (no GPU: matching and rewriting are
host logic; the fused graphs are executed in tests/test_gpu_fx.py).

Patterns and rules: "llm-fusion-compiler", pattern matcher (linear chains,
priority-based selection, no double fusion) and "LLMBoost", pattern matcher
(RMSNorm recognised as an op and by its reduce/rsqrt structure; the one-user
guard, whose negative case is tested here as the page's negative lit test
does)."""
import operator

import pytest
import torch

from gemm_epilogue_fuse_amd import fx as lfx
import fx_models as M


def trace(model, *inputs):
    from torch.fx.passes.shape_prop import ShapeProp
    gm = torch.fx.symbolic_trace(model)
    ShapeProp(gm).propagate(*inputs)
    return gm


def fused_targets(gm):
    return [n.target.__name__ for n in gm.graph.nodes if n.op == "call_function" and n.target.__name__.startswith("fused_")]


def compute_nodes(gm):
    return [n for n in gm.graph.nodes if n.op in ("call_module", "call_method", "call_function")
            and not (n.op == "call_function" and n.target.__name__.startswith("fused_"))
            and n.target is not operator.getitem]


def x16(*shape):
    return torch.randn(*shape).half()


def test_rmsnorm_linear_bias_gelu_becomes_one_call():
    m = M.RmsLinearGelu().half()
    gm, applied = lfx.fuse_graph(m, x16(2, 5, 64))
    assert applied == ["rmsnorm_gemm"]
    assert fused_targets(gm) == ["fused_rmsnorm_gemm"] and compute_nodes(gm) == []
    call = [n for n in gm.graph.nodes if n.op == "call_function"][0]
    x, gamma, eps, W, bias, act = call.args
    assert x.op == "placeholder" and eps == 1e-6 and act == "gelu_tanh"
    # the Linear weight [N, K] is stored [K, N], contiguous
    assert tuple(getattr(gm, W.target).shape) == (64, 48) and getattr(gm, W.target).is_contiguous()
    assert torch.equal(getattr(gm, W.target), m.proj.weight.detach().t())


def test_priority_picks_the_longest_pattern_and_no_node_twice():
    m = M.RmsLinearGelu().half()
    gm = trace(m, x16(3, 64))
    matches = lfx.find_fusion_matches(gm)
    assert [mm.pattern for mm in matches] == ["rmsnorm_gemm"]
    assert len(matches[0].nodes) == 3
    # the candidate set held the plain projection pattern too; it lost on priority
    seen = set()
    for mm in matches:
        assert not (set(mm.nodes) & seen)
        seen |= set(mm.nodes)


def test_structural_rmsnorm_is_recognised():
    m = M.DecomposedRmsQProj().half()
    gm, applied = lfx.fuse_graph(m, x16(4, 64))
    assert applied == ["rmsnorm_gemm"] and compute_nodes(gm) == []
    call = [n for n in gm.graph.nodes if n.op == "call_function"][0]
    assert call.args[2] == 1e-6 and call.args[4] is None and call.args[5] == "none"


def test_one_user_guard_keeps_a_shared_norm_unfused():
    m = M.SharedNormQKV().half()
    gm, applied = lfx.fuse_graph(m, x16(4, 64))
    # the norm feeds three projections: it is not fused; each projection with its bias still is
    assert applied == ["gemm_epilogue"] * 3
    assert [n.op for n in compute_nodes(gm)] == ["call_module"]  # the RMSNorm stays
    assert isinstance(gm.get_submodule(compute_nodes(gm)[0].target), torch.nn.RMSNorm)


def test_swiglu_block():
    m = M.SwiGluMlp().half()
    gm, applied = lfx.fuse_graph(m, x16(6, 64))
    assert sorted(applied) == ["gemm_epilogue", "rmsnorm_swiglu"]
    assert compute_nodes(gm) == []
    down = [n for n in gm.graph.nodes if n.op == "call_function" and n.target is lfx.fused_gemm][0]
    x, W, bias, residual, act = down.args
    assert residual.op == "placeholder" and act == "none" and bias is not None


def test_layernorm_linear_relu():
    gm, applied = lfx.fuse_graph(M.LnLinearRelu().half(), x16(5, 64))
    assert applied == ["layernorm_gemm"] and compute_nodes(gm) == []
    call = [n for n in gm.graph.nodes if n.op == "call_function"][0]
    assert call.args[3] == 1e-5 and call.args[-1] == "relu"


def test_prologue_bias_worked_example():
    gm, applied = lfx.fuse_graph(M.PrologueBias().half(), x16(16, 64))
    assert applied == ["prologue_bias_gemm"] and compute_nodes(gm) == []
    call = [n for n in gm.graph.nodes if n.op == "call_function"][0]
    assert call.args[-1] == "relu" and call.args[3] is None and call.args[4] is None


def test_epilogue_chain_and_exact_gelu_left_to_torch():
    gm, applied = lfx.fuse_graph(M.MatmulBiasActResidual().half(), x16(8, 64), x16(8, 48))
    assert applied == ["gemm_epilogue", "gemm_epilogue"]
    calls = [n for n in gm.graph.nodes if n.op == "call_function" and n.target is lfx.fused_gemm]
    first, second = calls
    assert first.args[4] == "silu" and first.args[3] is not None       # bias, SiLU and residual absorbed
    assert second.args[4] == "none" and second.args[3] is None         # exact GeLU is not fused
    assert [n.target for n in compute_nodes(gm)] == [torch.nn.functional.gelu]


def test_float32_graphs_are_left_alone():
    gm, applied = lfx.fuse_graph(M.SwiGluMlp(), torch.randn(4, 64))
    assert applied == [] and fused_targets(gm) == []


def test_fused_calls_refuse_host_tensors():
    gm, _ = lfx.fuse_graph(M.RmsLinearGelu().half(), x16(2, 64))
    with pytest.raises(ValueError, match="GPU"):
        gm(x16(2, 64))
