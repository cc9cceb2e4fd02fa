"""fp64 CPU oracle for the fused attention forward (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it, and it
imports nothing from the HIP path.

Source: "AttnFuse: A Composable DSL for Compiling Attentions to Fused GPU
Kernels" (arXiv 2609.13612).  The method reaches exactly the plain definition of
attention (the online-softmax recurrence in "2 Background / FlashAttention and
online softmax" is exact; the split-KV log-sum-exp merge in "4.2 Flash
Decoding" is exact), so this oracle computes that definition directly, with no
tiling and no online recurrence, in float64:

    out = softmax(mask(bias(RoPE(Q) . RoPE(K)^T * scale))) . V

built from the ten combinators of "3.1 The Researcher Interface"
(scaled_dot_product, rope, causal, sliding_window, full, block_sparse, alibi,
additive_bias, softmax; relu_attention is named there but never defined, so it
is not implemented).

Readings of points the pages leave open (each one is listed with its reason in
the design notes of the repository):
  * RoPE pairs dimension r with r + D/2 (NeoX convention, "4.1 Fused RoPE";
    the rotated half is "K with the two D-halves swapped", "7.2 Lessons
    Learned"), frequencies w_r = theta^(-2r/D) over the full head dim
    (RoFormer, the pages' reference [8]), angle = position * w_r.
  * Order: rotate, dot, scale, bias, mask, softmax, times V.
  * ALiBi adds slope_h * (p_k - p_q) (reference [7]); slopes are an input.
  * Sliding window W keeps 0 <= p_q - p_k < W when causal, |p_q - p_k| < W
    otherwise.
  * Grouped-query attention maps q-head h to kv-head h // (Hq / Hkv).
  * The saved statistic ("4.4 Backward Pass", L = m + log l) uses the natural
    log and is returned alongside the output.
  * A query row with no allowed key returns an all-zero output and
    lse = -inf.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def rope_frequencies(D: int, theta: float) -> np.ndarray:
    """w_r = theta^(-2r/D) for r = 0 .. D/2-1 (float64)."""
    if D % 2:
        raise ValueError("RoPE needs an even head dimension")
    r = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * r / D)


def rope_rotate(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate rows of ``x`` (shape [..., N, D]) by RoPE at ``positions`` [N].

    NeoX convention ("4.1 Fused RoPE"): for r < D/2 the pair
    (x[r], x[r + D/2]) is rotated by the angle a = p * w_r:
        x'[r]       = x[r] cos a - x[r + D/2] sin a
        x'[r + D/2] = x[r + D/2] cos a + x[r] sin a
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_frequencies(D, theta)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def allowed_mask(q_idx: np.ndarray, k_idx: np.ndarray, *, q_pos0: int = 0, k_pos0: int = 0,
                 causal: bool = False, window: int = 0, block_mask=None,
                 head: int = 0) -> np.ndarray:
    """Boolean [len(q_idx), len(k_idx)]: True where the key is visible.

    The AND of the active mask combinators:
      causal          p_k <= p_q
      sliding_window  0 <= p_q - p_k < W (causal) or |p_q - p_k| < W
      block_sparse    (i // bm, j // bn) is listed in the CSR BlockMask
                      ("4.3 Block-Sparse Attention")
    """
    q_idx = np.asarray(q_idx, dtype=np.int64)
    k_idx = np.asarray(k_idx, dtype=np.int64)
    pq = (q_pos0 + q_idx)[:, None]
    pk = (k_pos0 + k_idx)[None, :]
    ok = np.ones((q_idx.size, k_idx.size), dtype=bool)
    if causal:
        ok &= pk <= pq
    if window:
        dist = pq - pk
        if causal:
            ok &= (dist >= 0) & (dist < window)
        else:
            ok &= np.abs(dist) < window
    if block_mask is not None:
        row_ptr, col_idx, bm, bn = block_mask
        row_ptr = np.asarray(row_ptr)
        if row_ptr.ndim == 2:
            row_ptr = row_ptr[head]
        col_idx = np.asarray(col_idx)
        qb = q_idx // bm
        kb = k_idx // bn
        nkb = int(k_idx.max()) // bn + 1 if k_idx.size else 0
        for r, b in enumerate(qb):
            active = np.zeros(max(nkb, 1), dtype=bool)
            cols = col_idx[row_ptr[b]:row_ptr[b + 1]]
            cols = cols[cols < active.size]
            active[cols] = True
            ok[r] &= active[kb]
    return ok


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, scale: Optional[float] = None,
              rope_theta: Optional[float] = None, q_pos0: int = 0, k_pos0: int = 0,
              causal: bool = False, window: int = 0,
              alibi_slopes: Optional[np.ndarray] = None, bias: Optional[np.ndarray] = None,
              block_mask=None, rows: Optional[Sequence[int]] = None,
              heads: Optional[Sequence[tuple]] = None, row_block: int = 512):
    """Exact attention forward in float64.

    q [B, Hq, Nq, D], k and v [B, Hkv, Nk, D] (any real dtype, widened to
    float64).  ``bias`` broadcasts to [B, Hq, Nq, Nk].  ``block_mask`` is
    (row_ptr, col_idx, block_m, block_n) with row_ptr [nqb+1] shared by all
    heads or [Hq, nqb+1] per q-head.

    ``rows`` restricts the computation to those query indices and ``heads`` to
    those (b, h) pairs (other heads are left as NaN), so that single outputs of
    a large workload can be computed one by one.

    Returns (out [B, Hq, R, D], lse [B, Hq, R]) with R = len(rows) or Nq.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, Dk = k.shape
    if Dk != D or v.shape != k.shape or k.shape[0] != B or Hq % Hkv:
        raise ValueError("shape mismatch")
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    row_idx = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = row_idx.size
    k_idx = np.arange(Nk)
    out = np.full((B, Hq, R, D), np.nan)
    lse = np.full((B, Hq, R), np.nan)
    if bias is not None:
        bias = np.broadcast_to(np.asarray(bias, dtype=np.float64), (B, Hq, Nq, Nk))
    pairs = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    krot_cache = {}
    for b, h in pairs:
        kvh = h // group
        if (b, kvh) not in krot_cache:
            kk = k[b, kvh]
            if rope_theta is not None:
                kk = rope_rotate(kk, k_pos0 + k_idx, rope_theta)
            krot_cache = {(b, kvh): kk}
        kk = krot_cache[(b, kvh)]
        vv = v[b, kvh]
        for r0 in range(0, R, row_block):
            ri = row_idx[r0:r0 + row_block]
            qq = q[b, h, ri]
            if rope_theta is not None:
                qq = rope_rotate(qq, q_pos0 + ri, rope_theta)
            s = (qq @ kk.T) * scale
            if alibi_slopes is not None:
                slope = float(np.asarray(alibi_slopes, dtype=np.float64)[h])
                s = s + slope * ((k_pos0 + k_idx)[None, :] - (q_pos0 + ri)[:, None]).astype(np.float64)
            if bias is not None:
                s = s + bias[b, h][ri]
            ok = allowed_mask(ri, k_idx, q_pos0=q_pos0, k_pos0=k_pos0, causal=causal,
                              window=window, block_mask=block_mask, head=h)
            s = np.where(ok, s, -np.inf)
            any_ok = ok.any(axis=1)
            m = np.where(any_ok, s.max(axis=1), 0.0)
            e = np.exp(s - m[:, None])          # exp(-inf) = 0 for masked keys
            l = e.sum(axis=1)
            with np.errstate(divide="ignore", invalid="ignore"):
                o = (e @ vv) / l[:, None]
                ls = m + np.log(l)
            o[~any_ok] = 0.0
            ls[~any_ok] = -np.inf
            out[b, h, r0:r0 + ri.size] = o
            lse[b, h, r0:r0 + ri.size] = ls
    return out, lse

