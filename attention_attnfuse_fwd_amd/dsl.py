"""Composable attention front-end over the fused kernels.

Follows "AttnFuse: A Composable DSL for Compiling Attentions to Fused GPU
Kernels": "3.1 The Researcher Interface" (ten combinators composed in a
decorated Python function that is traced once), "3.2 From DSL to Kernel"
(a high-level IR of six node kinds, a SHA-1 signature over the graph's
structure used as the cache key, a fuse check of the canonical pattern and
a lowering to constants) and "3.3 Runtime Dispatch" (signature lookup of a
prepared launch, then the kernel; single-query and block-sparse calls take
their fast paths).

Everything here is host-side bookkeeping: the lowering target is the
library's variant descriptor (one field group per combinator) and the
specialised kernels are the C++ template instances already compiled into
libattnfuse.so, so "compiling" a program means validating it and fixing its
descriptor constants.  Tensors flow straight to ``ops.fwd`` / ``ops.bwd``.

    @attention
    def local_alibi(Q, K, V, w=1024):
        banded = sliding_window(causal(scaled_dot_product(Q, K)), w)
        return softmax(alibi(banded)) @ V

    out = local_alibi(q, k, v, alibi_slopes=slopes)          # traced on the first call
    out = local_alibi(q, k, v, w=256, alibi_slopes=slopes)   # another configuration
"""
from __future__ import annotations

import functools
import hashlib
import inspect
from dataclasses import dataclass
from typing import Callable, Dict, Optional, Tuple, Union

from . import ops

__all__ = [
    "attention", "run_attention", "trace", "fuse", "lower", "signature",
    "scaled_dot_product", "rope", "causal", "sliding_window", "full", "block_sparse", "alibi",
    "additive_bias", "softmax", "relu_attention",
    "TensorSym", "ScoreOp", "MaskOp", "BiasOp", "NormOp", "MatMulPV", "LaunchBundle",
    "DslError", "UnsupportedVariant",
]


class DslError(ValueError):
    """The program does not have the shape of one fused attention."""


class UnsupportedVariant(DslError):
    """A combinator that the pages name but the kernels do not implement."""


# ---------------------------------------------------------------------------
# High-level IR: six node kinds ("3.2 From DSL to Kernel")
# ---------------------------------------------------------------------------
class _Node:
    """Base of the IR nodes; ``@`` on a normalised score builds MatMulPV."""

    def __matmul__(self, other):
        if not isinstance(self, NormOp):
            raise DslError("only a normalised score (softmax(...)) can multiply V")
        if not isinstance(other, TensorSym):
            raise DslError("the value operand must be an input tensor")
        return MatMulPV(self, other)


@dataclass(frozen=True, eq=True)
class TensorSym(_Node):
    """An input tensor of the traced function (Q, K or V by position)."""
    role: str


@dataclass(frozen=True, eq=True)
class ScoreOp(_Node):
    """S = scale * op(Q) op(K)^T with op = RoPE or the identity."""
    q: TensorSym
    k: TensorSym
    rope: bool
    rope_theta: Optional[float]
    scale: Optional[float]


@dataclass(frozen=True, eq=True)
class MaskOp(_Node):
    """A mask on the score: causal, sliding window (width), full, block sparse."""
    src: _Node
    kind: str
    window: int = 0


@dataclass(frozen=True, eq=True)
class BiasOp(_Node):
    """An additive score modification: ALiBi slopes or a bias tensor."""
    src: _Node
    kind: str


@dataclass(frozen=True, eq=True)
class NormOp(_Node):
    """Row normalisation of the score: softmax (or relu, named but undefined)."""
    src: _Node
    kind: str


@dataclass(frozen=True, eq=True)
class MatMulPV(_Node):
    """O = P V."""
    p: NormOp
    v: TensorSym


# ---------------------------------------------------------------------------
# The ten combinators ("3.1 The Researcher Interface")
# ---------------------------------------------------------------------------
def _expect_tensor(x, role: str):
    if not isinstance(x, TensorSym):
        raise DslError(f"{role} must be an input tensor of the traced function")
    return x


def _expect_score(s):
    if not isinstance(s, (ScoreOp, MaskOp, BiasOp)):
        raise DslError("masks and biases apply to a score (rope(...) or scaled_dot_product(...))")
    return s


def scaled_dot_product(Q, K, scale: Optional[float] = None) -> ScoreOp:
    """S = scale * Q K^T (scale defaults to 1/sqrt(D))."""
    return ScoreOp(_expect_tensor(Q, "Q"), _expect_tensor(K, "K"), False, None,
                   None if scale is None else float(scale))


def rope(Q, K, theta: float = 10000.0, scale: Optional[float] = None) -> ScoreOp:
    """S = scale * RoPE(Q) RoPE(K)^T (NeoX half split, frequencies theta^(-2r/D))."""
    if not theta > 0:
        raise DslError("rope theta must be positive")
    return ScoreOp(_expect_tensor(Q, "Q"), _expect_tensor(K, "K"), True, float(theta),
                   None if scale is None else float(scale))


def causal(s) -> MaskOp:
    """Keys at positions after the query's are masked out."""
    return MaskOp(_expect_score(s), "causal")


def sliding_window(s, window: int) -> MaskOp:
    """Only keys within `window` positions of the query (including itself when
    combined with causal) are kept."""
    if int(window) < 1:
        raise DslError("sliding_window needs window >= 1")
    return MaskOp(_expect_score(s), "sliding_window", int(window))


def full(s) -> MaskOp:
    """No mask (every key visible)."""
    return MaskOp(_expect_score(s), "full")


def block_sparse(s) -> MaskOp:
    """Only the blocks of the call's ``block_mask`` (a CSR BlockMask) are visible."""
    return MaskOp(_expect_score(s), "block_sparse")


def alibi(s) -> BiasOp:
    """Adds slope_h * (key position - query position); slopes are the call's
    ``alibi_slopes``."""
    return BiasOp(_expect_score(s), "alibi")


def additive_bias(s) -> BiasOp:
    """Adds the call's ``bias`` tensor (fp32, broadcastable to [B, Hq, Nq, Nk])."""
    return BiasOp(_expect_score(s), "additive")


def softmax(s) -> NormOp:
    return NormOp(_expect_score(s), "softmax")


def relu_attention(s) -> NormOp:
    """Named by the pages but never defined: traced, then rejected by fuse()."""
    return NormOp(_expect_score(s), "relu")


# ---------------------------------------------------------------------------
# Tracing, signature, fuse check, lowering
# ---------------------------------------------------------------------------
def trace(fn: Callable, **static) -> MatMulPV:
    """Run `fn(Q, K, V, **static)` once on symbolic inputs and return its graph."""
    g = fn(TensorSym("Q"), TensorSym("K"), TensorSym("V"), **static)
    if not isinstance(g, MatMulPV):
        raise DslError("an attention program must return softmax(score) @ V")
    return g


def _chain(g: MatMulPV):
    """Nodes from the score to the output, in application order."""
    nodes = []
    n = g.p.src
    while isinstance(n, (MaskOp, BiasOp)):
        nodes.append(n)
        n = n.src
    if not isinstance(n, ScoreOp):
        raise DslError("the score must come from rope(...) or scaled_dot_product(...)")
    return n, list(reversed(nodes))


def _canonical(g: MatMulPV) -> str:
    score, mods = _chain(g)
    parts = [f"TensorSym({score.q.role})", f"TensorSym({score.k.role})",
             f"ScoreOp(rope={int(score.rope)},theta={score.rope_theta!r},scale={score.scale!r})"]
    for m in mods:
        if isinstance(m, MaskOp):
            parts.append(f"MaskOp({m.kind},{m.window})")
        else:
            parts.append(f"BiasOp({m.kind})")
    parts.append(f"NormOp({g.p.kind})")
    parts.append(f"MatMulPV(TensorSym({g.v.role}))")
    return "|".join(parts)


def signature(g: MatMulPV) -> str:
    """SHA-1 over the graph's structure (node kinds and static constants; no
    tensor data), the cache key of a prepared launch."""
    return hashlib.sha1(_canonical(g).encode()).hexdigest()


@dataclass(frozen=True)
class LaunchBundle:
    """Descriptor constants of one fused program (the lowered form)."""
    signature: str
    causal: bool
    window: int
    rope_theta: Optional[float]
    scale: Optional[float]
    alibi: bool
    bias: bool
    block_sparse: bool

    def fwd_kwargs(self) -> dict:
        return dict(causal=self.causal, window=self.window, rope_theta=self.rope_theta,
                    scale=self.scale)


def fuse(g: MatMulPV) -> Tuple[ScoreOp, list]:
    """Check the canonical pattern score -> masks / biases -> softmax -> @ V on
    the traced inputs (Q, K, V in that role) and return its parts."""
    if not isinstance(g, MatMulPV):
        raise DslError("an attention program must return softmax(score) @ V")
    score, mods = _chain(g)
    if (score.q.role, score.k.role, g.v.role) != ("Q", "K", "V"):
        raise DslError(f"operands must be (Q, K) for the score and V for the values, got "
                       f"({score.q.role}, {score.k.role}) and {g.v.role}")
    if g.p.kind == "relu":
        raise UnsupportedVariant("relu_attention is named by the pages but not defined; "
                                 "no kernel implements it")
    if g.p.kind != "softmax":
        raise DslError(f"unknown normalisation {g.p.kind}")
    seen = set()
    for m in mods:
        key = (type(m).__name__, m.kind)
        if key in seen and key != ("MaskOp", "full") and key != ("MaskOp", "causal"):
            raise DslError(f"{m.kind} applied twice")
        seen.add(key)
    return score, mods


def lower(g: MatMulPV) -> LaunchBundle:
    """Fold the graph into descriptor constants (masks intersect, biases add)."""
    score, mods = fuse(g)
    is_causal = any(isinstance(m, MaskOp) and m.kind == "causal" for m in mods)
    window = next((m.window for m in mods if isinstance(m, MaskOp) and m.kind == "sliding_window"), 0)
    return LaunchBundle(
        signature=signature(g), causal=is_causal, window=window,
        rope_theta=score.rope_theta if score.rope else None, scale=score.scale,
        alibi=any(isinstance(m, BiasOp) and m.kind == "alibi" for m in mods),
        bias=any(isinstance(m, BiasOp) and m.kind == "additive" for m in mods),
        block_sparse=any(isinstance(m, MaskOp) and m.kind == "block_sparse" for m in mods))


# Prepared launches by signature, shared by every program ("3.3 Runtime Dispatch").
_BUNDLES: Dict[str, LaunchBundle] = {}


def _prepare(g: MatMulPV) -> LaunchBundle:
    b = lower(g)
    return _BUNDLES.setdefault(b.signature, b)


def _runtime_operands(b: LaunchBundle, alibi_slopes, bias, block_mask) -> dict:
    for need, val, name in ((b.alibi, alibi_slopes, "alibi_slopes"), (b.bias, bias, "bias"),
                            (b.block_sparse, block_mask, "block_mask")):
        if need and val is None:
            raise DslError(f"the program uses {name}; pass it to the call")
        if not need and val is not None:
            raise DslError(f"the program does not use {name}")
    return dict(alibi_slopes=alibi_slopes, bias=bias, block_mask=block_mask)


def run_attention(bundle_or_graph: Union[LaunchBundle, MatMulPV], q, k, v, *, alibi_slopes=None,
                  bias=None, block_mask=None, q_pos0: int = 0, k_pos0: int = 0,
                  return_lse: bool = False, out=None):
    """Launch a prepared program on tensors: one fused kernel (or the split-KV
    decode pair for a single query row)."""
    b = bundle_or_graph if isinstance(bundle_or_graph, LaunchBundle) else _prepare(bundle_or_graph)
    rt = _runtime_operands(b, alibi_slopes, bias, block_mask)
    return ops.fwd(q, k, v, q_pos0=q_pos0, k_pos0=k_pos0, return_lse=return_lse, out=out,
                   **b.fwd_kwargs(), **rt)


class AttentionProgram:
    """A decorated attention function: traced once per static configuration
    (its keyword arguments other than the runtime operands), then dispatched
    by signature."""

    _RUNTIME = ("alibi_slopes", "bias", "block_mask", "q_pos0", "k_pos0", "return_lse", "out")

    def __init__(self, fn: Callable):
        self.fn = fn
        self._by_config: Dict[tuple, LaunchBundle] = {}
        functools.update_wrapper(self, fn)

    def bundle(self, **static) -> LaunchBundle:
        key = tuple(sorted(static.items()))
        b = self._by_config.get(key)
        if b is None:
            b = _prepare(trace(self.fn, **static))
            self._by_config[key] = b
        return b

    def graph(self, **static) -> MatMulPV:
        return trace(self.fn, **static)

    def __call__(self, q, k, v, **kwargs):
        runtime = {n: kwargs.pop(n) for n in self._RUNTIME if n in kwargs}
        return run_attention(self.bundle(**kwargs), q, k, v, **runtime)

    def backward(self, q, k, v, out, dout, lse, *, alibi_slopes=None, bias=None, block_mask=None,
                 q_pos0: int = 0, k_pos0: int = 0, workspace=None, **static):
        """Gradients (dq, dk, dv) of the same program ("4.4 Backward Pass")."""
        b = self.bundle(**static)
        _runtime_operands(b, alibi_slopes, bias, block_mask)
        return ops.bwd(q, k, v, out, dout, lse, causal=b.causal, window=b.window,
                       rope_theta=b.rope_theta, scale=b.scale, alibi_slopes=alibi_slopes,
                       bias=bias, block_mask=block_mask, q_pos0=q_pos0, k_pos0=k_pos0,
                       workspace=workspace)


def attention(fn: Callable) -> AttentionProgram:
    """Decorator: ``@attention def f(Q, K, V, **config): ... return softmax(s) @ V``."""
    params = list(inspect.signature(fn).parameters)
    if len(params) < 3:
        raise DslError("an attention program takes (Q, K, V, ...)")
    return AttentionProgram(fn)
