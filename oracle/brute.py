"""Pure-Python brute-force attention for tiny shapes (TEST INFRASTRUCTURE ONLY).

A second, independently written rendering of the same definition as
``oracle.attention`` ("AttnFuse: A Composable DSL for Compiling Attentions to
Fused GPU Kernels", "3.1 The Researcher Interface" combinators, "4.1 Fused
RoPE" for the rotation): every score, weight and output element is computed by
explicit loops with the ``math`` module, one (batch, head, query) at a time.
It shares no code with ``oracle.attention`` and is meant for inputs of a few
hundred elements.
"""
from __future__ import annotations

import math


def _rotate_vector(x, pos, theta):
    """RoPE of one vector at one position: pair (r, r + D/2), angle pos*theta^(-2r/D)."""
    D = len(x)
    half = D // 2
    y = [0.0] * D
    for r in range(half):
        a = pos * math.pow(theta, -2.0 * r / D)
        c, s = math.cos(a), math.sin(a)
        y[r] = x[r] * c - x[r + half] * s
        y[r + half] = x[r + half] * c + x[r] * s
    return y


def _visible(pq, pk, i, j, causal, window, block):
    if causal and pk > pq:
        return False
    if window:
        d = pq - pk
        if causal:
            if not (0 <= d < window):
                return False
        elif abs(d) >= window:
            return False
    if block is not None:
        row_ptr, col_idx, bm, bn = block
        rb, cb = i // bm, j // bn
        if cb not in list(col_idx[row_ptr[rb]:row_ptr[rb + 1]]):
            return False
    return True


def attention_brute(q, k, v, scale=None, rope_theta=None, q_pos0=0, k_pos0=0, causal=False,
                    window=0, alibi_slopes=None, bias=None, block_mask=None):
    """Loops over (b, h, i); q, k, v are nested sequences [B][H][N][D].

    ``bias`` is a nested [B][Hq][Nq][Nk] sequence or None; ``block_mask`` is
    (row_ptr, col_idx, bm, bn) with a flat row_ptr shared by every head, or a
    per-head list of row_ptr rows.
    Returns (out [B][Hq][Nq][D], lse [B][Hq][Nq]) as nested lists.
    """
    B = len(q)
    Hq = len(q[0])
    Nq = len(q[0][0])
    D = len(q[0][0][0])
    Hkv = len(k[0])
    Nk = len(k[0][0])
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = []
    lse = []
    for b in range(B):
        ob, lb = [], []
        for h in range(Hq):
            kvh = h // group
            blk = None
            if block_mask is not None:
                rp, ci, bm, bn = block_mask
                if len(rp) and hasattr(rp[0], "__len__"):
                    rp = rp[h]
                blk = (list(rp), list(ci), bm, bn)
            oh, lh = [], []
            for i in range(Nq):
                pq = q_pos0 + i
                qi = [float(x) for x in q[b][h][i]]
                if rope_theta is not None:
                    qi = _rotate_vector(qi, pq, rope_theta)
                scores = []
                for j in range(Nk):
                    pk = k_pos0 + j
                    if not _visible(pq, pk, i, j, causal, window, blk):
                        continue
                    kj = [float(x) for x in k[b][kvh][j]]
                    if rope_theta is not None:
                        kj = _rotate_vector(kj, pk, rope_theta)
                    s = 0.0
                    for d in range(D):
                        s += qi[d] * kj[d]
                    s *= scale
                    if alibi_slopes is not None:
                        s += float(alibi_slopes[h]) * (pk - pq)
                    if bias is not None:
                        s += float(bias[b][h][i][j])
                    scores.append((j, s))
                if not scores:
                    oh.append([0.0] * D)
                    lh.append(-math.inf)
                    continue
                m = max(s for _, s in scores)
                w = [(j, math.exp(s - m)) for j, s in scores]
                total = sum(x for _, x in w)
                o = [0.0] * D
                for j, x in w:
                    vj = v[b][kvh][j]
                    for d in range(D):
                        o[d] += x * float(vj[d])
                oh.append([x / total for x in o])
                lh.append(m + math.log(total))
            ob.append(oh)
            lb.append(lh)
        out.append(ob)
        lse.append(lb)
    return out, lse
