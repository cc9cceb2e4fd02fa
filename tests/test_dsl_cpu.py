"""Host-side checks of the attention front-end (tracing, the six-node IR,
SHA-1 signatures, the fuse check and the lowering to descriptor constants),
after "3.1 The Researcher Interface", "3.2 From DSL to Kernel" and "3.3
Runtime Dispatch".  No GPU: nothing here launches a kernel."""
import hashlib

import pytest

import attention_attnfuse_fwd_amd.dsl as af


@af.attention
def llama_attn(Q, K, V, theta=500000.0):
    s = af.rope(Q, K, theta=theta)
    s = af.causal(s)
    return af.softmax(s) @ V


def test_ten_combinators_are_exposed():
    names = ["scaled_dot_product", "rope", "causal", "sliding_window", "full", "block_sparse",
             "alibi", "additive_bias", "softmax", "relu_attention"]
    for n in names:
        assert callable(getattr(af, n)), n
    assert set(names) <= set(af.__all__)


def test_trace_builds_the_six_node_chain():
    g = llama_attn.graph()
    assert isinstance(g, af.MatMulPV) and isinstance(g.v, af.TensorSym) and g.v.role == "V"
    assert isinstance(g.p, af.NormOp) and g.p.kind == "softmax"
    m = g.p.src
    assert isinstance(m, af.MaskOp) and m.kind == "causal"
    s = m.src
    assert isinstance(s, af.ScoreOp) and s.rope and s.rope_theta == 500000.0
    assert (s.q.role, s.k.role) == ("Q", "K")


def test_lowering_of_the_llama_program():
    b = llama_attn.bundle()
    assert (b.causal, b.window, b.rope_theta, b.scale) == (True, 0, 500000.0, None)
    assert not (b.alibi or b.bias or b.block_sparse)
    assert b.fwd_kwargs() == dict(causal=True, window=0, rope_theta=500000.0, scale=None)


def test_signature_is_sha1_of_structure_only():
    @af.attention
    def same(Q, K, V):
        return af.softmax(af.causal(af.rope(Q, K, theta=500000.0))) @ V

    g1, g2 = llama_attn.graph(), same.graph()
    assert af.signature(g1) == af.signature(g2)
    assert af.signature(g1) == hashlib.sha1(af._canonical(g1).encode()).hexdigest()
    assert len(af.signature(g1)) == 40
    # a different static constant or structure changes the key
    assert af.signature(llama_attn.graph(theta=10000.0)) != af.signature(g1)

    @af.attention
    def windowed(Q, K, V, w=256):
        return af.softmax(af.sliding_window(af.causal(af.rope(Q, K, theta=500000.0)), w)) @ V

    assert af.signature(windowed.graph()) != af.signature(g1)
    assert af.signature(windowed.graph(w=128)) != af.signature(windowed.graph())


def test_configurations_are_traced_once_and_bundles_shared():
    calls = []

    @af.attention
    def counted(Q, K, V, w=64):
        calls.append(w)
        return af.softmax(af.sliding_window(af.scaled_dot_product(Q, K), w)) @ V

    b1 = counted.bundle()
    b2 = counted.bundle()
    b3 = counted.bundle(w=32)
    assert b1 is b2 and b1 is not b3 and calls == [64, 32]
    assert (b1.window, b3.window, b1.causal) == (64, 32, False)

    @af.attention
    def counted_twin(Q, K, V):
        return af.softmax(af.sliding_window(af.scaled_dot_product(Q, K), 64)) @ V

    assert counted_twin.bundle() is b1  # same signature -> the same prepared launch


def test_alibi_window_bias_and_block_sparse_lowering():
    @af.attention
    def alibi_sw(Q, K, V):
        return af.softmax(af.alibi(af.sliding_window(af.causal(af.scaled_dot_product(Q, K, scale=0.1)), 1024))) @ V

    b = alibi_sw.bundle()
    assert (b.causal, b.window, b.rope_theta, b.scale, b.alibi, b.bias) == (True, 1024, None, 0.1, True, False)

    @af.attention
    def biased(Q, K, V):
        return af.softmax(af.additive_bias(af.full(af.scaled_dot_product(Q, K)))) @ V

    b = biased.bundle()
    assert (b.causal, b.window, b.bias, b.alibi) == (False, 0, True, False)

    @af.attention
    def bigbird(Q, K, V):
        return af.softmax(af.block_sparse(af.rope(Q, K, theta=10000.0))) @ V

    b = bigbird.bundle()
    assert b.block_sparse and b.rope_theta == 10000.0 and not b.causal


def test_runtime_operands_are_checked_against_the_program():
    @af.attention
    def alibi_prog(Q, K, V):
        return af.softmax(af.alibi(af.scaled_dot_product(Q, K))) @ V

    b = alibi_prog.bundle()
    with pytest.raises(af.DslError, match="alibi_slopes"):
        af._runtime_operands(b, None, None, None)
    with pytest.raises(af.DslError, match="bias"):
        af._runtime_operands(b, [1.0], object(), None)
    assert af._runtime_operands(b, [1.0], None, None)["alibi_slopes"] == [1.0]


def test_fuse_rejects_programs_that_are_not_one_attention():
    with pytest.raises(af.DslError):  # no normalisation before @ V
        af.trace(lambda Q, K, V: af.causal(af.rope(Q, K)) @ V)
    with pytest.raises(af.DslError):  # values must be V
        af.lower(af.trace(lambda Q, K, V: af.softmax(af.scaled_dot_product(Q, K)) @ Q))
    with pytest.raises(af.DslError):  # score operands swapped
        af.lower(af.trace(lambda Q, K, V: af.softmax(af.scaled_dot_product(K, Q)) @ V))
    with pytest.raises(af.DslError):  # a mask on a tensor, not a score
        af.trace(lambda Q, K, V: af.softmax(af.causal(Q)) @ V)
    with pytest.raises(af.DslError):  # a mask after the normalisation
        af.trace(lambda Q, K, V: af.causal(af.softmax(af.rope(Q, K))) @ V)
    with pytest.raises(af.DslError):  # the program must end in @ V
        af.trace(lambda Q, K, V: af.softmax(af.rope(Q, K)))
    with pytest.raises(af.DslError):  # two windows
        af.lower(af.trace(lambda Q, K, V: af.softmax(af.sliding_window(af.sliding_window(
            af.rope(Q, K), 8), 4)) @ V))
    with pytest.raises(af.DslError):
        af.sliding_window(af.rope(af.TensorSym("Q"), af.TensorSym("K")), 0)
    with pytest.raises(af.DslError):
        af.rope(af.TensorSym("Q"), af.TensorSym("K"), theta=0.0)


def test_relu_attention_is_traced_then_rejected():
    g = af.trace(lambda Q, K, V: af.relu_attention(af.scaled_dot_product(Q, K)) @ V)
    assert g.p.kind == "relu"
    with pytest.raises(af.UnsupportedVariant):
        af.lower(g)


def test_backward_checks_runtime_operands_before_any_launch():
    @af.attention
    def sparse(Q, K, V):
        return af.softmax(af.block_sparse(af.scaled_dot_product(Q, K))) @ V

    with pytest.raises(af.DslError, match="block_mask"):
        sparse.backward(None, None, None, None, None, None)
