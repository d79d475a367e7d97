"""Graph-level fusion: find the fusible patterns in a torch.fx graph and
rewrite each into one libfuse call.

The pages' compiler half, built on top of the kernels:

* "llm-fusion-compiler", pattern matcher: a topological walk of the dataflow
  graph, linear-chain detection, patterns with priority-based selection, and
  no double fusion (each op used at most once); its API is
  ``find_fusion_matches`` then ``apply_fusion``, kept here.
* "LLMBoost", pattern matcher: RMSNorm is recognised both as the library op
  and by structure (a reduction of x*x over the last axis, then a normalise
  containing rsqrt), and the one-user safety guard skips the fusion when the
  normalised tensor has more than one consumer (fusing would recompute or
  buffer it).

Patterns, highest priority first (a chain stops at any intermediate with more
than one user):

  rmsnorm_swiglu      RMSNorm -> two projections g, u -> SiLU(g) * u
                      (the normalised tensor has exactly those two users)
  rmsnorm_gemm        RMSNorm -> projection [-> + bias] [-> act]
  layernorm_gemm      LayerNorm -> projection [-> + bias] [-> act]
  prologue_bias_gemm  (x + b[K]) -> projection [-> + bias] [-> act] [-> + residual]
  gemm_epilogue       projection [-> + bias] [-> act] [-> + residual]

A projection is ``nn.Linear``, ``F.linear`` with a parameter weight, or a 2-D
``matmul``/``mm`` against a parameter [K, N].  act is ReLU, GeLU with
``approximate="tanh"`` or SiLU (an exact-erf GeLU is left to torch).  Only
fp16 and bf16 activations are rewritten; the graph is shape-propagated with
example inputs to tell a bias [N] from a residual [.., N] and to read dtypes.
Linear weights are stored [N, K]; the rewrite snapshots each as a contiguous
[K, N] buffer on the module (an inference graph: later weight updates are not
seen).  The fused calls run on the GPU only, through the C ABI; on any other
device they raise.
"""
from __future__ import annotations

import operator
from dataclasses import dataclass, field

import torch
import torch.fx as fx
import torch.nn.functional as F

from . import gemm_epilogue, gemm_prologue_bias, layernorm_gemm, rmsnorm_gemm, rmsnorm_gemm_swiglu

PRIORITY = {"rmsnorm_swiglu": 100, "rmsnorm_gemm": 90, "layernorm_gemm": 85, "prologue_bias_gemm": 70,
            "gemm_epilogue": 50}
FUSED_DTYPES = (torch.float16, torch.bfloat16)


@dataclass
class Match:
    pattern: str
    out: fx.Node                  # the node whose value the fused call replaces
    nodes: list                   # every node the fused call absorbs (out included)
    parts: dict = field(default_factory=dict)

    @property
    def priority(self) -> int:
        return PRIORITY[self.pattern]


# ----------------------------------------------------------------------------- fused calls (run time)

def _rows(x):
    """x [..., K] as a contiguous 2-D [rows, K] view, and the leading shape."""
    lead = x.shape[:-1]
    return x.reshape(-1, x.shape[-1]).contiguous(), lead


def fused_gemm(x, W, bias, residual, act):
    a, lead = _rows(x)
    r = None if residual is None else residual.reshape(-1, residual.shape[-1]).contiguous()
    y = gemm_epilogue(a, W, bias, r, act)
    return y.reshape(*lead, W.shape[1])


def fused_rmsnorm_gemm(x, gamma, eps, W, bias, act):
    a, lead = _rows(x)
    return rmsnorm_gemm(a, gamma, W, eps, bias, act).reshape(*lead, W.shape[1])


def fused_layernorm_gemm(x, gamma, beta, eps, W, bias, act):
    a, lead = _rows(x)
    return layernorm_gemm(a, gamma, W, eps, beta, bias, act).reshape(*lead, W.shape[1])


def fused_prologue_bias_gemm(x, abias, W, bias, residual, act):
    a, lead = _rows(x)
    r = None if residual is None else residual.reshape(-1, residual.shape[-1]).contiguous()
    return gemm_prologue_bias(a, abias, W, bias, r, act).reshape(*lead, W.shape[1])


def fused_rmsnorm_swiglu(x, gamma, eps, Wg, Wu):
    a, lead = _rows(x)
    return rmsnorm_gemm_swiglu(a, gamma, Wg, Wu, eps).reshape(*lead, Wg.shape[1])


# ----------------------------------------------------------------------------- recognisers

def _meta(n):
    return n.meta.get("tensor_meta") if isinstance(n, fx.Node) else None


def _shape(n):
    m = _meta(n)
    return tuple(m.shape) if m is not None else None


def _is_fn(n, *fns):
    return isinstance(n, fx.Node) and n.op == "call_function" and n.target in fns


def _is_method(n, *names):
    return isinstance(n, fx.Node) and n.op == "call_method" and n.target in names


def _module(gm, n):
    return gm.get_submodule(n.target) if isinstance(n, fx.Node) and n.op == "call_module" else None


def _single_user(n):
    return len(n.users) == 1


def _strip_casts(n):
    """Skip dtype casts (.to, .float, .type_as) back to the tensor they cast."""
    while _is_method(n, "to", "float", "type_as", "half", "bfloat16"):
        n = n.args[0]
    return n


def _param_node(gm, n):
    """The tensor behind a get_attr node (a parameter or buffer), else None."""
    if isinstance(n, fx.Node) and n.op == "get_attr":
        obj = gm
        for part in n.target.split("."):
            obj = getattr(obj, part)
        return obj if isinstance(obj, torch.Tensor) else None
    return None


def _projection(gm, n):
    """(input node, weight [K,N] spec, bias spec) of a projection node, else None.
    A weight spec is ("kn", tensor) for a [K,N] parameter or ("nk", tensor) for
    an [N,K] one (nn.Linear, F.linear); a bias spec is a tensor or None."""
    mod = _module(gm, n)
    if isinstance(mod, torch.nn.Linear):
        return n.args[0], ("nk", mod.weight), mod.bias
    if _is_fn(n, F.linear):
        w = _param_node(gm, n.args[1])
        b = n.args[2] if len(n.args) > 2 else n.kwargs.get("bias")
        bt = _param_node(gm, b) if b is not None else None
        if w is None or (b is not None and bt is None):
            return None
        return n.args[0], ("nk", w), bt
    if _is_fn(n, torch.matmul, operator.matmul, torch.mm):
        w = _param_node(gm, n.args[1])
        if w is not None and w.dim() == 2:
            return n.args[0], ("kn", w), None
    return None


def _act(gm, n):
    """The activation name a node applies to its single input, else None."""
    mod = _module(gm, n)
    if isinstance(mod, torch.nn.ReLU) or _is_fn(n, F.relu, torch.relu) or _is_method(n, "relu"):
        return "relu"
    if isinstance(mod, torch.nn.SiLU) or _is_fn(n, F.silu):
        return "silu"
    if isinstance(mod, torch.nn.GELU) and mod.approximate == "tanh":
        return "gelu_tanh"
    if _is_fn(n, F.gelu) and n.kwargs.get("approximate", "none") == "tanh":
        return "gelu_tanh"
    return None


def _add_other(n, x):
    """For an add node with x as one operand, the other operand."""
    if _is_fn(n, operator.add, torch.add) and len(n.args) == 2 and not n.kwargs:
        a, b = n.args
        if a is x:
            return b
        if b is x:
            return a
    return None


def _mul_operands(n):
    if _is_fn(n, operator.mul, torch.mul) and len(n.args) == 2:
        return n.args
    return None


def _rmsnorm(gm, n):
    """(x, gamma tensor, eps) if n computes RMSNorm over the last axis."""
    mod = _module(gm, n)

    def default_eps(x):
        # torch's RMSNorm without an eps uses the machine epsilon of the input type
        m = _meta(x)
        return float(torch.finfo(m.dtype).eps) if m is not None else None
    if isinstance(mod, torch.nn.RMSNorm) and mod.weight is not None and len(mod.normalized_shape) == 1:
        eps = mod.eps if mod.eps is not None else default_eps(n.args[0])
        return (n.args[0], mod.weight, float(eps)) if eps is not None else None
    if _is_fn(n, F.rms_norm):
        x, shape = n.args[0], n.args[1]
        w = _param_node(gm, n.args[2] if len(n.args) > 2 else n.kwargs.get("weight"))
        eps = n.args[3] if len(n.args) > 3 else n.kwargs.get("eps")
        if eps is None:
            eps = default_eps(x)
        if w is not None and len(shape) == 1 and isinstance(eps, float):
            return x, w, eps
        return None
    # structural form: gamma * (x * rsqrt(mean(x^2, -1, keepdim) + eps)), either order
    ops = _mul_operands(_strip_casts(n))
    if ops is None:
        return None
    for w_node, inner in (ops, ops[::-1]):
        w = _param_node(gm, w_node)
        inner_ops = _mul_operands(_strip_casts(inner)) if w is not None else None
        if inner_ops is None:
            continue
        for x, r in (inner_ops, inner_ops[::-1]):
            found = _rsqrt_mean_square(r, x)
            if found is not None:
                return _strip_casts(x), w, found
    return None


def _rsqrt_mean_square(r, x):
    """eps if r = rsqrt(mean(x^2 over the last axis, keepdim) + eps), else None."""
    if not (_is_fn(r, torch.rsqrt) or _is_method(r, "rsqrt")):
        return None
    s = r.args[0]
    if not _is_fn(s, operator.add, torch.add) or len(s.args) != 2:
        return None
    var, eps = s.args
    if isinstance(var, float):
        var, eps = eps, var
    if not isinstance(eps, float):
        return None
    if _is_method(var, "mean") or _is_fn(var, torch.mean):
        dim = var.args[1] if len(var.args) > 1 else var.kwargs.get("dim")
        if dim not in (-1, [-1], (-1,)) or not var.kwargs.get("keepdim", False):
            return None
        sq = var.args[0]
        base = _strip_casts(x)
        if (_is_method(sq, "pow") or _is_fn(sq, torch.pow, operator.pow)) and sq.args[1] == 2:
            if _strip_casts(sq.args[0]) is base:
                return eps
        ops = _mul_operands(sq)
        if ops is not None and _strip_casts(ops[0]) is base and _strip_casts(ops[1]) is base:
            return eps
    return None


def _layernorm(gm, n):
    """(x, gamma, beta, eps) if n is LayerNorm over the last axis with a gamma."""
    mod = _module(gm, n)
    if isinstance(mod, torch.nn.LayerNorm) and mod.weight is not None and len(mod.normalized_shape) == 1:
        return n.args[0], mod.weight, mod.bias, float(mod.eps)
    if _is_fn(n, F.layer_norm):
        shape = n.args[1]
        w = _param_node(gm, n.args[2] if len(n.args) > 2 else n.kwargs.get("weight"))
        bn = n.args[3] if len(n.args) > 3 else n.kwargs.get("bias")
        b = _param_node(gm, bn) if bn is not None else None
        eps = n.args[4] if len(n.args) > 4 else n.kwargs.get("eps", 1e-5)
        if w is not None and len(shape) == 1 and (bn is None or b is not None):
            return n.args[0], w, b, float(eps)
    return None


# ----------------------------------------------------------------------------- matching

def _epilogue_chain(gm, proj, has_bias, allow_residual=True):
    """Extend a projection node along its single-user chain: + bias [N] (unless
    the projection has its own), then an activation, then + residual [same
    shape].  Returns (nodes, bias node, act, residual node)."""
    nodes, cur = [proj], proj
    bias = act = residual = None
    out_shape = _shape(proj)
    if not has_bias and _single_user(cur):
        u = next(iter(cur.users))
        other = _add_other(u, cur)
        if other is not None and out_shape is not None and _shape(other) == (out_shape[-1],):
            bias = other
            nodes.append(u)
            cur = u
    if _single_user(cur):
        u = next(iter(cur.users))
        a = _act(gm, u)
        if a is not None:
            act = a
            nodes.append(u)
            cur = u
    if allow_residual and _single_user(cur):
        u = next(iter(cur.users))
        other = _add_other(u, cur)
        if other is not None and out_shape is not None and _shape(other) == out_shape:
            residual = other
            nodes.append(u)
    return nodes, bias, act, residual


def _fusible_dtype(n):
    m = _meta(n)
    return m is not None and m.dtype in FUSED_DTYPES


def find_fusion_matches(gm: fx.GraphModule):
    """Every fusible pattern in the graph, walked in topological order, with
    overlaps resolved by priority (then graph order): no node is absorbed by
    two matches.  The graph must carry shape metadata (``ShapeProp``)."""
    cands = []
    for n in gm.graph.nodes:
        p = _projection(gm, n)
        if p is None or not _fusible_dtype(n):
            continue
        x = p[0]
        has_bias = p[2] is not None
        nodes, bias, act, residual = _epilogue_chain(gm, n, has_bias)
        base = dict(x=x, weight=p[1], pbias=p[2], bias=bias, act=act, residual=residual)
        cands.append(Match("gemm_epilogue", nodes[-1], nodes, base))
        # a norm or an input bias in front of the projection, if it feeds only it
        if isinstance(x, fx.Node) and _single_user(x):
            rms = _rmsnorm(gm, x)
            if rms is not None:
                en, eb, ea, _ = _epilogue_chain(gm, n, has_bias, allow_residual=False)
                cands.append(Match("rmsnorm_gemm", en[-1], [x] + en,
                                   dict(base, x=rms[0], gamma=rms[1], eps=rms[2], bias=eb, act=ea, residual=None)))
            ln = _layernorm(gm, x)
            if ln is not None:
                en, eb, ea, _ = _epilogue_chain(gm, n, has_bias, allow_residual=False)
                cands.append(Match("layernorm_gemm", en[-1], [x] + en,
                                   dict(base, x=ln[0], gamma=ln[1], beta=ln[2], eps=ln[3], bias=eb, act=ea,
                                        residual=None)))
            for a_node in (x.args[:2] if _is_fn(x, operator.add, torch.add) and len(x.args) == 2 else ()):
                other = _add_other(x, a_node)
                K = _shape(x)[-1] if _shape(x) else None
                ab = _param_node(gm, other)
                if ab is not None and K is not None and tuple(ab.shape) == (K,) and _shape(a_node) == _shape(x):
                    cands.append(Match("prologue_bias_gemm", nodes[-1], [x] + nodes,
                                       dict(base, x=a_node, abias=ab)))
                    break
    # the SwiGLU gate/up pair: a norm with exactly two projection users
    for n in gm.graph.nodes:
        rms = _rmsnorm(gm, n)
        if rms is None or len(n.users) != 2 or not _fusible_dtype(n):
            continue
        projs = [u for u in n.users if _projection(gm, u) is not None and _projection(gm, u)[2] is None]
        if len(projs) != 2 or not all(_single_user(p) for p in projs):
            continue
        for g, u in (projs, projs[::-1]):
            s = next(iter(g.users))
            if _act(gm, s) != "silu" or not _single_user(s):
                continue
            m = next(iter(s.users))
            ops = _mul_operands(m)
            if ops is not None and set(ops) == {s, u} and next(iter(u.users)) is m:
                cands.append(Match("rmsnorm_swiglu", m, [n, g, u, s, m],
                                   dict(x=rms[0], gamma=rms[1], eps=rms[2], wg=_projection(gm, g)[1],
                                        wu=_projection(gm, u)[1])))
                break
    order = {n: i for i, n in enumerate(gm.graph.nodes)}
    cands.sort(key=lambda m: (-m.priority, order[m.out]))
    taken, out = set(), []
    for m in cands:
        if any(n in taken for n in m.nodes):
            continue
        taken.update(m.nodes)
        out.append(m)
    out.sort(key=lambda m: order[m.out])
    return out


# ----------------------------------------------------------------------------- rewriting

def _const(gm, graph, tensor, prefix):
    """A get_attr node for `tensor`, registered on gm under a fresh name."""
    i = 0
    while hasattr(gm, "%s%d" % (prefix, i)):
        i += 1
    name = "%s%d" % (prefix, i)
    gm.register_buffer(name, tensor)
    return graph.get_attr(name)


def _weight_kn(gm, graph, spec):
    kind, w = spec
    t = w.detach()
    t = t.t().contiguous() if kind == "nk" else t.contiguous()
    return _const(gm, graph, t, "_libfuse_w")


def _tensor_const(gm, graph, t, prefix):
    return None if t is None else _const(gm, graph, t.detach().contiguous(), prefix)


def apply_fusion(gm: fx.GraphModule, matches) -> tuple:
    """Rewrite each match into one call of the fused op; returns (gm, the
    list of pattern names applied).  Absorbed nodes are removed."""
    graph = gm.graph
    applied = []
    repl = {}  # output node of an applied match -> its fused call
    for m in matches:
        # inputs may be outputs of matches already rewritten
        p = {k: repl.get(v, v) if isinstance(v, fx.Node) else v for k, v in m.parts.items()}
        with graph.inserting_before(m.out):
            if m.pattern == "rmsnorm_swiglu":
                args = (p["x"], _tensor_const(gm, graph, p["gamma"], "_libfuse_g"), p["eps"],
                        _weight_kn(gm, graph, p["wg"]), _weight_kn(gm, graph, p["wu"]))
                new = graph.call_function(fused_rmsnorm_swiglu, args)
            else:
                W = _weight_kn(gm, graph, p["weight"])
                # a bias add after the projection, or the projection's own bias
                bias = p["bias"] if p["bias"] is not None else _tensor_const(gm, graph, p["pbias"], "_libfuse_b")
                if m.pattern == "gemm_epilogue":
                    new = graph.call_function(fused_gemm, (p["x"], W, bias, p["residual"], p["act"] or "none"))
                elif m.pattern == "rmsnorm_gemm":
                    new = graph.call_function(fused_rmsnorm_gemm, (p["x"], _tensor_const(gm, graph, p["gamma"],
                                                                                         "_libfuse_g"),
                                                                   p["eps"], W, bias, p["act"] or "none"))
                elif m.pattern == "layernorm_gemm":
                    new = graph.call_function(fused_layernorm_gemm, (
                        p["x"], _tensor_const(gm, graph, p["gamma"], "_libfuse_g"),
                        _tensor_const(gm, graph, p["beta"], "_libfuse_be"), p["eps"], W, bias, p["act"] or "none"))
                else:
                    new = graph.call_function(fused_prologue_bias_gemm, (
                        p["x"], _tensor_const(gm, graph, p["abias"], "_libfuse_ab"), W, bias, p["residual"],
                        p["act"] or "none"))
        new.meta = dict(m.out.meta)
        m.out.replace_all_uses_with(new)
        repl[m.out] = new
        applied.append(m.pattern)
    graph.eliminate_dead_code()
    graph.lint()
    gm.recompile()
    return gm, applied


def fuse_graph(module: torch.nn.Module, *example_inputs):
    """Trace `module`, propagate shapes with `example_inputs`, and rewrite every
    fusible pattern into libfuse calls.  Returns (GraphModule, applied patterns)."""
    from torch.fx.passes.shape_prop import ShapeProp
    gm = fx.symbolic_trace(module)
    ShapeProp(gm).propagate(*example_inputs)
    return apply_fusion(gm, find_fusion_matches(gm))
