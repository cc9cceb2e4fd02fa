"""fp64 CPU oracle for the attention backward (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it, and it
imports nothing from the HIP path.

Source: "AttnFuse: A Composable DSL for Compiling Attentions to Fused GPU
Kernels", "4.4 Backward Pass": the backward of the same forward
(softmax(mask(bias(RoPE(Q) . RoPE(K)^T * scale))) . V), with the forward
saving one statistic per query row.  The pages give the kernel decomposition
(a row-reduction pre-pass, a key/value-gradient pass, a query-gradient pass);
the result they reach is the plain gradient, which this oracle computes
directly by the chain rule on the full score matrix, in float64, for the
scalar  L = sum(out * dout):

    S  = scale * Q' K'^T (+ ALiBi / additive bias), masked to -inf
    P  = softmax(S) row by row          (all-zero for a row with no key)
    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))      (the softmax Jacobian)
    dQ' = scale * dS K' ,  dK' = scale * dS^T Q'
    dQ = R_q^T dQ' ,  dK = R_k^T dK'    (R^T rotates by the negative angle)

With grouped-query attention the gradients of a kv-head sum over its q-heads.
Pinned by finite differences of the forward oracle (tests/test_oracle_backward.py).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import allowed_mask, rope_rotate


def attention_backward(q, k, v, dout, *, scale: Optional[float] = None,
                       rope_theta: Optional[float] = None, q_pos0: int = 0, k_pos0: int = 0,
                       causal: bool = False, window: int = 0,
                       alibi_slopes: Optional[np.ndarray] = None,
                       bias: Optional[np.ndarray] = None, block_mask=None):
    """Gradients (dq [B,Hq,Nq,D], dk [B,Hkv,Nk,D], dv [B,Hkv,Nk,D]) of
    sum(attention(q, k, v, ...) * dout), float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = k.shape
    if do.shape != q.shape or v.shape != k.shape or Hq % Hkv:
        raise ValueError("shape mismatch")
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    q_idx = np.arange(Nq)
    k_idx = np.arange(Nk)
    if bias is not None:
        bias = np.broadcast_to(np.asarray(bias, dtype=np.float64), (B, Hq, Nq, Nk))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for kvh in range(Hkv):
            kr = k[b, kvh]
            if rope_theta is not None:
                kr = rope_rotate(kr, k_pos0 + k_idx, rope_theta)
            vv = v[b, kvh]
            dkr = np.zeros((Nk, D))
            for h in range(kvh * group, (kvh + 1) * group):
                qr = q[b, h]
                if rope_theta is not None:
                    qr = rope_rotate(qr, q_pos0 + q_idx, rope_theta)
                s = (qr @ kr.T) * scale
                if alibi_slopes is not None:
                    slope = float(np.asarray(alibi_slopes, dtype=np.float64)[h])
                    s = s + slope * ((k_pos0 + k_idx)[None, :] - (q_pos0 + q_idx)[:, None])
                if bias is not None:
                    s = s + bias[b, h]
                ok = allowed_mask(q_idx, k_idx, q_pos0=q_pos0, k_pos0=k_pos0, causal=causal,
                                  window=window, block_mask=block_mask, head=h)
                s = np.where(ok, s, -np.inf)
                any_ok = ok.any(axis=1)
                m = np.where(any_ok, s.max(axis=1), 0.0)
                e = np.exp(s - m[:, None])
                l = e.sum(axis=1)
                p = np.where(any_ok[:, None], e / np.where(any_ok, l, 1.0)[:, None], 0.0)
                g = do[b, h]
                dv[b, kvh] += p.T @ g
                dp = g @ vv.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dqr = scale * (ds @ kr)
                dkr += scale * (ds.T @ qr)
                if rope_theta is not None:
                    dqr = rope_rotate(dqr, -(q_pos0 + q_idx), rope_theta)
                dq[b, h] = dqr
            if rope_theta is not None:
                dkr = rope_rotate(dkr, -(k_pos0 + k_idx), rope_theta)
            dk[b, kvh] = dkr
    return dq, dk, dv
