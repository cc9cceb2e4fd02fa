"""Helpers for the GPU parity tests: device copies of seeded inputs and the
tolerance checks (bf16 I/O: max |err| <= 2e-2 and mean |err| <= 2e-3;
fp32: max |err| <= 1e-4)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np

import oracle
import workloads

BF16_MAX = 2e-2
BF16_MEAN = 2e-3
FP32_MAX = 1e-4


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def to_dev(arr: np.ndarray, dtype: str, device="cuda"):
    """bf16 bit patterns (uint16) or float32 numpy array -> device tensor."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def dev_inputs(inp: workloads.Inputs, device="cuda"):
    w = inp.w
    return (to_dev(inp.q_dev, w.dtype, device), to_dev(inp.k_dev, w.dtype, device),
            to_dev(inp.v_dev, w.dtype, device))


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """Assert the bar for `dtype`; returns (max_err, mean_err)."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    where = np.unravel_index(int(err.argmax()), err.shape) if err.size else None
    msg = f"{what}: max {mx:.3e} at {where} (got {got[where] if where else None}, ref {ref[where] if where else None}), mean {mean:.3e}"
    log(msg)
    if dtype == "bf16":
        assert mx <= BF16_MAX and mean <= BF16_MEAN, msg
    else:
        assert mx <= FP32_MAX, msg
    return mx, mean


def check_lse(got: np.ndarray, ref: np.ndarray, tol: float, what: str = ""):
    both_inf = np.isneginf(got) & np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf pattern differs"
    err = np.abs(np.where(both_inf, 0.0, got) - np.where(both_inf, 0.0, ref))
    log(f"{what}: lse max err {float(err.max()) if err.size else 0:.3e}")
    assert float(err.max() if err.size else 0) <= tol, what


def oracle_all_heads(q, k, v, B: int, Hq: int, workers: int = 0, **kw):
    """The oracle over every (batch, q-head) pair, one pair per task on a thread
    pool (numpy's BLAS and ufuncs release the GIL; BLAS runs one thread per
    task).  Same result as one ``oracle.attention`` call over all heads."""
    from threadpoolctl import threadpool_limits
    workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    pairs = [(b, h) for b in range(B) for h in range(Hq)]

    def one(bh):
        o, l = oracle.attention(q, k, v, heads=[bh], **kw)
        return bh, o[bh], l[bh]

    out = lse = None
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            for (b, h), o, l in ex.map(one, pairs):
                if out is None:
                    out = np.empty((B, Hq) + o.shape, dtype=np.float64)
                    lse = np.empty((B, Hq) + l.shape, dtype=np.float64)
                out[b, h], lse[b, h] = o, l
    return out, lse
