"""Pins for the CPU oracle, written as functions of an oracle module ``O``.

Each pin checks the oracle against something other than itself: a closed form,
an invariant the pages state, a library routine (PyTorch's
``scaled_dot_product_attention`` in float64 on the CPU, ``scipy``'s
``logsumexp``) or an independent brute force.  ``test_oracle_pins.py`` runs
them on the real oracle; ``test_oracle_mutants.py`` runs them on copies of the
oracle with one plausible mistake planted and requires that some pin fails.

Page references are to "AttnFuse: A Composable DSL for Compiling Attentions to
Fused GPU Kernels".
"""
from __future__ import annotations

import math

import numpy as np
import torch
from scipy.special import logsumexp

import workloads

RTOL = 1e-10
ATOL = 1e-10


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa(q, k, v, mask=None, scale=None):
    """Library attention in float64 on the CPU (K/V repeated for GQA)."""
    G = q.shape[1] // k.shape[1]
    tq = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))
    tk = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64)).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).repeat_interleave(G, dim=1)
    tm = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale)
    return o.numpy()


# ----------------------------------------------------------------------------
# RoPE ("2 Background / Rotary Position Embeddings", "4.1 Fused RoPE")
# ----------------------------------------------------------------------------

def pin_rope_d2_rotation(O):
    """D=2: w_0 = 1, so RoPE is the plane rotation by angle p (counter-clockwise)."""
    p = np.array([0.0, 1.0, 7.0, 1000.0, 32768.0])
    y = O.rope_rotate(np.tile([1.0, 0.0], (p.size, 1)), p, 10000.0)
    np.testing.assert_allclose(y, np.stack([np.cos(p), np.sin(p)], 1), rtol=0, atol=1e-12)
    y = O.rope_rotate(np.tile([0.0, 1.0], (p.size, 1)), p, 10000.0)
    np.testing.assert_allclose(y, np.stack([-np.sin(p), np.cos(p)], 1), rtol=0, atol=1e-12)


def pin_rope_half_split_pairing(O):
    """D=4, theta=100: dim 1 pairs with dim 3 (halves, NeoX) at w_1 = theta^(-1/2) = 0.1."""
    p = np.array([3.0, 11.0])
    e1 = np.tile([0.0, 1.0, 0.0, 0.0], (2, 1))
    y = O.rope_rotate(e1, p, 100.0)
    exp = np.stack([np.zeros(2), np.cos(0.1 * p), np.zeros(2), np.sin(0.1 * p)], 1)
    np.testing.assert_allclose(y, exp, rtol=0, atol=1e-12)
    e0 = np.tile([1.0, 0.0, 0.0, 0.0], (2, 1))
    y = O.rope_rotate(e0, p, 100.0)
    exp = np.stack([np.cos(p), np.zeros(2), np.sin(p), np.zeros(2)], 1)
    np.testing.assert_allclose(y, exp, rtol=0, atol=1e-12)


def pin_rope_group_property(O):
    """R(a) R(b) = R(a + b), identity at position 0, and norms are kept."""
    rng = _rng(11)
    x = rng.standard_normal((6, 128))
    a = np.array([0, 1, 5, 4096, 30000, 32767], dtype=np.float64)
    b = np.array([0, 2, 9, 1, 768, 1], dtype=np.float64)
    two = O.rope_rotate(O.rope_rotate(x, a, 5e5), b, 5e5)
    one = O.rope_rotate(x, a + b, 5e5)
    np.testing.assert_allclose(two, one, rtol=0, atol=1e-9)
    np.testing.assert_allclose(O.rope_rotate(x, np.zeros(6), 5e5), x, rtol=0, atol=0)
    np.testing.assert_allclose(np.linalg.norm(one, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)


def pin_rope_toeplitz(O):
    """Constant q and k rows: RoPE scores depend only on j - i ("2 Background", RoPE)."""
    rng = _rng(12)
    u, w = rng.standard_normal(16), rng.standard_normal(16)
    n = 24
    qr = O.rope_rotate(np.tile(u, (n, 1)), np.arange(n), 10000.0)
    kr = O.rope_rotate(np.tile(w, (n, 1)), np.arange(n), 10000.0)
    s = qr @ kr.T
    for d in range(-n + 1, n):
        diag = np.diagonal(s, offset=d)
        np.testing.assert_allclose(diag, np.full_like(diag, diag[0]), rtol=0, atol=1e-9)
    # and not a constant matrix: different offsets give different scores
    assert abs(s[0, 1] - s[0, 2]) > 1e-6


def pin_rope_shift_invariance(O):
    """Adding c to both q_pos0 and k_pos0 leaves the attention output unchanged."""
    rng = _rng(13)
    q, k, v = (rng.standard_normal((1, 2, 20, 8)) for _ in range(3))
    for causal in (True, False):
        a, la = O.attention(q, k, v, rope_theta=10000.0, causal=causal)
        b, lb = O.attention(q, k, v, rope_theta=10000.0, causal=causal, q_pos0=1000, k_pos0=1000)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-9)
        np.testing.assert_allclose(la, lb, rtol=0, atol=1e-9)
    # and RoPE is not a no-op on the output
    c, _ = O.attention(q, k, v, rope_theta=None, causal=True)
    assert np.max(np.abs(a - c)) > 1e-3


# ----------------------------------------------------------------------------
# Plain attention against the library routine (RoPE and ALiBi off)
# ----------------------------------------------------------------------------

def _explicit_mask(Nq, Nk, causal=False, window=0, block=None):
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    m = np.ones((Nq, Nk), dtype=bool)
    if causal:
        m &= j <= i
    if window:
        m &= ((i - j >= 0) & (i - j < window)) if causal else (np.abs(i - j) < window)
    if block is not None:
        row_ptr, col_idx, bm, bn = block
        nqb = -(-Nq // bm)
        nkb = -(-Nk // bn)
        dense = np.zeros((nqb, nkb), dtype=bool)
        for r in range(nqb):
            dense[r, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
        m &= np.kron(dense, np.ones((bm, bn), dtype=bool))[:Nq, :Nk]
    return m


def pin_matches_library_sdpa(O):
    rng = _rng(14)
    B, Hq, Hkv, Nq, Nk, D = 2, 4, 2, 37, 37, 16
    q = rng.standard_normal((B, Hq, Nq, D))
    k = rng.standard_normal((B, Hkv, Nk, D))
    v = rng.standard_normal((B, Hkv, Nk, D))
    rp, ci = workloads.bigbird_csr(-(-Nq // 8), -(-Nk // 8), seed=5, n_random=1)
    cases = [
        dict(),
        dict(causal=True),
        dict(causal=True, window=5),
        dict(window=4),
        dict(block_mask=(rp, ci, 8, 8)),
        dict(block_mask=(rp, ci, 8, 8), causal=True),
    ]
    for kw in cases:
        out, _ = O.attention(q, k, v, **kw)
        mask = _explicit_mask(Nq, Nk, kw.get("causal", False), kw.get("window", 0),
                              kw.get("block_mask"))
        ref = _sdpa(q, k, v, mask=mask)
        np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-9, err_msg=str(kw))
    # additive bias = float attn_mask of the library routine
    bias = rng.standard_normal((B, Hq, Nq, Nk))
    out, _ = O.attention(q, k, v, bias=bias)
    np.testing.assert_allclose(out, _sdpa(q, k, v, mask=bias), rtol=1e-9, atol=1e-9)
    # a non-default scale
    out, _ = O.attention(q, k, v, scale=0.3, causal=True)
    ref = _sdpa(q, k, v, mask=_explicit_mask(Nq, Nk, True), scale=0.3)
    np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-9)


def pin_default_scale_closed_form(O):
    """Two keys, D=4: s0 = <q,k0>/sqrt(4), s1 = 0 -> weight of key 0 is the logistic of s0."""
    q = np.array([1.0, 2.0, -1.0, 0.5]).reshape(1, 1, 1, 4)
    k = np.array([[0.5, 1.0, 1.0, 2.0], [0.0, 0.0, 0.0, 0.0]]).reshape(1, 1, 2, 4)
    v = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]]).reshape(1, 1, 2, 4)
    out, lse = O.attention(q, k, v)
    s0 = (0.5 + 2.0 - 1.0 + 1.0) / 2.0
    w0 = 1.0 / (1.0 + math.exp(-s0))
    np.testing.assert_allclose(out[0, 0, 0], [w0, 1 - w0, 0, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0, 0], math.log(math.exp(s0) + 1.0), rtol=1e-14)


def pin_lse_against_logsumexp(O):
    """lse_i = log sum_j exp(s_ij) over visible keys ("4.4 Backward Pass": L = m + log l)."""
    rng = _rng(15)
    q, k, v = (rng.standard_normal((1, 2, 19, 8)) for _ in range(3))
    _, lse = O.attention(q, k, v, causal=True, scale=0.4)
    s = torch.matmul(torch.from_numpy(q), torch.from_numpy(k).transpose(-1, -2)).numpy() * 0.4
    s = np.where(np.tril(np.ones((19, 19), dtype=bool)), s, -np.inf)
    np.testing.assert_allclose(lse, logsumexp(s, axis=-1), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# Special cases with closed forms
# ----------------------------------------------------------------------------

def pin_causal_row0_is_v0(O):
    rng = _rng(16)
    q, k, v = (rng.standard_normal((2, 3, 17, 8)) for _ in range(3))
    out, lse = O.attention(q, k, v, rope_theta=10000.0, causal=True)
    np.testing.assert_array_equal(out[:, :, 0], v[:, :, 0])


def pin_window_one_is_identity(O):
    rng = _rng(17)
    q, k, v = (rng.standard_normal((1, 2, 13, 8)) for _ in range(3))
    for causal in (True, False):
        out, _ = O.attention(q, k, v, rope_theta=10000.0, causal=causal, window=1)
        np.testing.assert_allclose(out, v, rtol=0, atol=1e-15)


def pin_window_covering_all_is_causal(O):
    rng = _rng(18)
    q, k, v = (rng.standard_normal((1, 2, 21, 8)) for _ in range(3))
    a, la = O.attention(q, k, v, rope_theta=500.0, causal=True)
    for W in (21, 22, 100):
        b, lb = O.attention(q, k, v, rope_theta=500.0, causal=True, window=W)
        np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(la, lb)
    c, _ = O.attention(q, k, v, rope_theta=500.0, causal=True, window=20)
    assert np.max(np.abs(c[:, :, 20] - a[:, :, 20])) > 1e-6


def pin_window_width_counts_keys(O):
    """Q = 0 (uniform scores): causal window W averages exactly min(i+1, W) keys."""
    rng = _rng(19)
    N, W = 30, 7
    v = rng.standard_normal((1, 1, N, 4))
    q = np.zeros((1, 1, N, 4))
    k = rng.standard_normal((1, 1, N, 4))
    out, lse = O.attention(q, k, v, causal=True, window=W, rope_theta=10000.0)
    for i in range(N):
        lo = max(0, i - W + 1)
        np.testing.assert_allclose(out[0, 0, i], v[0, 0, lo:i + 1].mean(0), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, 0, i], math.log(i + 1 - lo), rtol=0, atol=1e-12)
    out, lse = O.attention(q, k, v, causal=False, window=W)
    for i in range(N):
        lo, hi = max(0, i - W + 1), min(N, i + W)
        np.testing.assert_allclose(out[0, 0, i], v[0, 0, lo:hi].mean(0), rtol=0, atol=1e-12)


def pin_q_zero_prefix_mean(O):
    """Q = 0: every score is 0 (RoPE of 0 is 0), so row i is the mean of V[0..i] and lse = ln(i+1)."""
    rng = _rng(20)
    N = 25
    q = np.zeros((1, 2, N, 8))
    k, v = (rng.standard_normal((1, 1, N, 8)) for _ in range(2))
    out, lse = O.attention(q, k, v, rope_theta=10000.0, causal=True)
    ref = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    for h in range(2):
        np.testing.assert_allclose(out[0, h], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], np.log(np.arange(1, N + 1)), rtol=0, atol=1e-12)


def pin_alibi_geometric_closed_form(O):
    """Q = 0, causal, ALiBi slope m, V_j = j: weights r^(i-j) with r = e^-m.

    O_i = sum_t (i - t) r^t / sum_t r^t (t = 0..i), summed with the
    arithmetico-geometric series formulas rather than term by term.
    """
    N, H = 40, 4
    slopes = np.array([0.25, 1.5, 0.6, 3.0])
    q = np.zeros((1, H, N, 4))
    k = np.ones((1, 1, N, 4))          # one kv head shared by the four q heads (GQA)
    v = np.tile(np.arange(N, dtype=np.float64)[:, None], (1, 4))[None, None]
    out, lse = O.attention(q, k, v, causal=True, alibi_slopes=slopes)
    for h, m in enumerate(slopes):
        r = math.exp(-m)
        for i in range(N):
            s0 = (1 - r ** (i + 1)) / (1 - r)
            s1 = r * (1 - (i + 1) * r ** i + i * r ** (i + 1)) / (1 - r) ** 2
            np.testing.assert_allclose(out[0, h, i, 0], (i * s0 - s1) / s0, rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(lse[0, h, i], math.log(s0), rtol=1e-11, atol=1e-11)


def pin_alibi_limits(O):
    rng = _rng(21)
    q, k, v = (rng.standard_normal((1, 3, 15, 8)) for _ in range(3))
    a, _ = O.attention(q, k, v, causal=True, rope_theta=1e4)
    b, _ = O.attention(q, k, v, causal=True, rope_theta=1e4, alibi_slopes=np.zeros(3))
    np.testing.assert_array_equal(a, b)
    c, _ = O.attention(q, k, v, causal=True, rope_theta=1e4, alibi_slopes=np.full(3, 200.0))
    np.testing.assert_allclose(c, v, rtol=0, atol=1e-12)


def pin_block_sparse_structure(O):
    """All blocks = full attention; diagonal blocks only = independent per-block attention."""
    rng = _rng(22)
    N, bs = 32, 8
    q, k, v = (rng.standard_normal((1, 2, N, 8)) for _ in range(3))
    nb = N // bs
    full_rp = np.arange(0, nb * nb + 1, nb, dtype=np.int32)
    full_ci = np.tile(np.arange(nb, dtype=np.int32), nb)
    a, la = O.attention(q, k, v, rope_theta=1e4)
    b, lb = O.attention(q, k, v, rope_theta=1e4, block_mask=(full_rp, full_ci, bs, bs))
    np.testing.assert_array_equal(a, b)
    diag_rp = np.arange(nb + 1, dtype=np.int32)
    diag_ci = np.arange(nb, dtype=np.int32)
    c, _ = O.attention(q, k, v, block_mask=(diag_rp, diag_ci, bs, bs))
    for r in range(nb):
        sl = slice(r * bs, (r + 1) * bs)
        ref = _sdpa(q[:, :, sl], k[:, :, sl], v[:, :, sl])
        np.testing.assert_allclose(c[:, :, sl], ref, rtol=1e-12, atol=1e-12)


def pin_block_sparse_per_head_and_empty_rows(O):
    """Per-head CSR rows; a row with no active block gives O = 0 and lse = -inf."""
    rng = _rng(23)
    N, bs, H = 24, 8, 2
    q, k, v = (rng.standard_normal((1, H, N, 4)) for _ in range(3))
    # head 0: row 1 empty; head 1: every row sees block 2 only
    rp = np.array([[0, 1, 1, 3], [3, 4, 5, 6]], dtype=np.int32)
    ci = np.array([0, 0, 2, 2, 2, 2], dtype=np.int32)
    out, lse = O.attention(q, k, v, block_mask=(rp, ci, bs, bs))
    np.testing.assert_array_equal(out[0, 0, 8:16], 0.0)
    assert np.all(np.isneginf(lse[0, 0, 8:16]))
    ref = _sdpa(q[:, 1:2], k[:, 1:2, 16:24], v[:, 1:2, 16:24])
    np.testing.assert_allclose(out[:, 1:2], ref, rtol=1e-12, atol=1e-12)
    ref0 = _sdpa(q[:, :1, :8], k[:, :1, :8], v[:, :1, :8])
    np.testing.assert_allclose(out[:, :1, :8], ref0, rtol=1e-12, atol=1e-12)


def pin_gqa_equals_repeated_heads(O):
    rng = _rng(24)
    q = rng.standard_normal((2, 8, 11, 8))
    k, v = (rng.standard_normal((2, 2, 11, 8)) for _ in range(2))
    a, la = O.attention(q, k, v, rope_theta=1e4, causal=True)
    b, lb = O.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), rope_theta=1e4,
                        causal=True)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def pin_rows_and_heads_subsets(O):
    """Computing selected rows / heads one by one gives the same values as the whole."""
    rng = _rng(25)
    q = rng.standard_normal((2, 4, 33, 8))
    k, v = (rng.standard_normal((2, 2, 33, 8)) for _ in range(2))
    kw = dict(rope_theta=1e4, causal=True, window=9, alibi_slopes=np.array([.1, .2, .3, .4]))
    a, la = O.attention(q, k, v, **kw)
    rows = [0, 5, 17, 32]
    b, lb = O.attention(q, k, v, rows=rows, heads=[(1, 3), (0, 0)], **kw)
    for bb, hh in [(1, 3), (0, 0)]:
        np.testing.assert_allclose(b[bb, hh], a[bb, hh, rows], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lb[bb, hh], la[bb, hh, rows], rtol=1e-13, atol=1e-13)
    assert np.isnan(b[1, 0]).all()


def pin_decode_is_last_prefill_row(O):
    """A single query at position P over a cache at positions 0..P-1 equals row P of a
    causal prefill of length P+1 whose own key (column P) is hidden by a -inf bias."""
    rng = _rng(26)
    P, D = 50, 16
    q1 = rng.standard_normal((1, 4, 1, D))
    k, v = (rng.standard_normal((1, 2, P, D)) for _ in range(2))
    a, la = O.attention(q1, k, v, rope_theta=5e5, q_pos0=P, k_pos0=0)
    # the same as a prefill whose query sits at index P of a P+1 long sequence, with the
    # extra key made invisible by a -inf additive bias
    qf = np.zeros((1, 4, P + 1, D))
    qf[:, :, P] = q1[:, :, 0]
    kf = np.concatenate([k, np.zeros((1, 2, 1, D))], axis=2)
    vf = np.concatenate([v, np.zeros((1, 2, 1, D))], axis=2)
    bias = np.zeros((1, 4, P + 1, P + 1))
    bias[..., P] = -np.inf
    b, lb = O.attention(qf, kf, vf, rope_theta=5e5, causal=True, bias=bias, rows=[P])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(la, lb, rtol=1e-12, atol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def brute_compare(O, B, Hq, Hkv, Nq, Nk, D, seed, rope, causal, window, alibi, bias,
                  block, q_pos0, k_pos0):
    """Oracle vs the pure-Python brute force on one tiny random case."""
    rng = _rng(seed)
    q = rng.standard_normal((B, Hq, Nq, D))
    k = rng.standard_normal((B, Hkv, Nk, D))
    v = rng.standard_normal((B, Hkv, Nk, D))
    kw = dict(causal=causal, window=window, q_pos0=q_pos0, k_pos0=k_pos0)
    if rope:
        kw["rope_theta"] = 100.0
    if alibi:
        kw["alibi_slopes"] = rng.uniform(0.05, 1.0, size=Hq)
    if bias:
        kw["bias"] = rng.standard_normal((B, Hq, Nq, Nk))
    if block:
        bs = 4
        nqb, nkb = -(-Nq // bs), -(-Nk // bs)
        rp, ci = workloads.random_csr(nqb, nkb, 0.6, seed=seed + 1, n_heads=Hq)
        kw["block_mask"] = (rp, ci, bs, bs)
    out, lse = O.attention(q, k, v, **kw)
    bkw = dict(kw)
    if block:
        bkw["block_mask"] = ([list(r) for r in rp], list(ci), bs, bs)
    if bias:
        bkw["bias"] = kw["bias"].tolist()
    bo, bl = O.attention_brute(q.tolist(), k.tolist(), v.tolist(), **bkw)
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(lse, np.array(bl), rtol=1e-10, atol=1e-10)
