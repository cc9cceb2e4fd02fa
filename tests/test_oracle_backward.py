"""Pins of the backward oracle ("4.4 Backward Pass"): its gradients must equal
central finite differences of the forward oracle, for every mask and score
combinator, with GQA, ragged shapes and position offsets; planted mistakes in
a copy of it must be caught by those differences."""
import os
import types

import numpy as np
import pytest

import oracle

VARIANTS = {
    "plain": dict(),
    "rope": dict(rope_theta=10.0),
    "causal": dict(causal=True),
    "rope_causal_offsets": dict(rope_theta=7.0, causal=True, q_pos0=3, k_pos0=2),
    "window": dict(window=2),
    "causal_window": dict(causal=True, window=3, rope_theta=5.0),
    "alibi": dict(alibi=True, causal=True),
    "bias": dict(bias=True),
    "block": dict(block=True, rope_theta=9.0),
    "empty_rows": dict(causal=True, q_pos0=0, k_pos0=3),  # rows 0..2 see no key
}
B, HQ, HKV, NQ, NK, D = 1, 4, 2, 5, 6, 4


def _inputs(seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, HQ, NQ, D))
    k = rng.standard_normal((B, HKV, NK, D))
    v = rng.standard_normal((B, HKV, NK, D))
    do = rng.standard_normal((B, HQ, NQ, D))
    return rng, q, k, v, do


def _kwargs(var, rng):
    kw = {key: val for key, val in var.items() if key not in ("alibi", "bias", "block")}
    if var.get("alibi"):
        kw["alibi_slopes"] = np.array([0.5, 0.25, 0.125, 0.0625])
    if var.get("bias"):
        kw["bias"] = rng.standard_normal((B, HQ, NQ, NK))
    if var.get("block"):
        # 2x2 blocks; block rows list different key blocks (one row lists none)
        kw["block_mask"] = (np.array([0, 2, 3, 3]), np.array([0, 2, 1]), 2, 2)
    return kw


def _finite_differences(q, k, v, do, kw, h=1e-5):
    def loss(qq, kk, vv):
        out, _ = oracle.attention(qq, kk, vv, **kw)
        return float(np.sum(out * do))
    grads = []
    for x_idx in range(3):
        xs = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(xs[x_idx])
        for idx in np.ndindex(g.shape):
            plus = [a.copy() for a in xs]
            minus = [a.copy() for a in xs]
            plus[x_idx][idx] += h
            minus[x_idx][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


def _check(backward, var, seed=0):
    rng, q, k, v, do = _inputs(seed)
    kw = _kwargs(var, rng)
    got = backward(q, k, v, do, **kw)
    want = _finite_differences(q, k, v, do, kw)
    return max(float(np.max(np.abs(a - b))) for a, b in zip(got, want))


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_backward_matches_finite_differences(name):
    assert _check(oracle.attention_backward, VARIANTS[name]) < 1e-7


def test_empty_rows_have_zero_query_gradient():
    rng, q, k, v, do = _inputs(1)
    dq, _, _ = oracle.attention_backward(q, k, v, do, causal=True, k_pos0=3)
    assert np.all(dq[:, :, :3] == 0.0)


def test_gqa_equals_repeated_heads_summed():
    rng, q, k, v, do = _inputs(2)
    kw = dict(rope_theta=11.0, causal=True)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, **kw)
    g = HQ // HKV
    k_rep, v_rep = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    dq2, dk2, dv2 = oracle.attention_backward(q, k_rep, v_rep, do, **kw)
    assert np.allclose(dq, dq2, atol=1e-12)
    assert np.allclose(dk, dk2.reshape(B, HKV, g, NK, D).sum(axis=2), atol=1e-12)
    assert np.allclose(dv, dv2.reshape(B, HKV, g, NK, D).sum(axis=2), atol=1e-12)


# ---- planted mistakes in a private copy of oracle/backward.py ----
SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "backward.py")
MUTATIONS = {
    "softmax_jacobian_missing_row_term": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    "dv_only_last_head": ("dv[b, kvh] += p.T @ g", "dv[b, kvh] = p.T @ g"),
    "dq_missing_scale": ("dqr = scale * (ds @ kr)", "dqr = ds @ kr"),
    "dk_unrotated_with_positive_angle": ("dkr = rope_rotate(dkr, -(k_pos0 + k_idx), rope_theta)",
                                         "dkr = rope_rotate(dkr, (k_pos0 + k_idx), rope_theta)"),
    "dq_not_unrotated": ("dqr = rope_rotate(dqr, -(q_pos0 + q_idx), rope_theta)", "dqr = dqr"),
    "dk_only_last_head": ("dkr += scale * (ds.T @ qr)", "dkr = scale * (ds.T @ qr)"),
    "dp_uses_keys": ("dp = g @ vv.T", "dp = g @ kr.T"),
    "alibi_sign": ("(k_pos0 + k_idx)[None, :] - (q_pos0 + q_idx)[:, None]",
                   "(q_pos0 + q_idx)[:, None] - (k_pos0 + k_idx)[None, :]"),
}


def _mutant(old, new):
    src = open(SRC).read()
    assert old in src, old
    src = src.replace(old, new).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("backward_mutant")
    exec(compile(src, "backward_mutant", "exec"), mod.__dict__)
    return mod.attention_backward


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_finite_differences_catch_mutation(name):
    bwd = _mutant(*MUTATIONS[name])
    errs = []
    for var in ("rope_causal_offsets", "alibi", "plain"):
        try:
            errs.append(_check(bwd, VARIANTS[var]))
        except Exception:
            errs.append(np.inf)
    assert max(errs) > 1e-4, (name, errs)
