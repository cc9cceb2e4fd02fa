"""Seeded synthetic inputs for the fused attention forward and split-KV decode.

This module only draws and formats inputs.  It holds none of the attention
arithmetic: the CPU oracle (``oracle/``) and the HIP path
(``attention_attnfuse_fwd_amd``) both take what it produces and compute on
their own.

Workloads follow the shapes the AttnFuse pages evaluate on (Llama-3-8B /
Llama-3-70B attention geometry in "6.3 KV-Cache Decoding" and "6.5 End-to-End",
a BigBird mask in "4.3 Block-Sparse Attention", sliding window and ALiBi in
"6.1 Forward Head-to-Head on Ampere").  The pages use no dataset: every input
here is iid N(0, 1) from ``numpy.random.default_rng(seed)``.

Recipe (same for every config):
  * Q, K, V are drawn as float32 ``standard_normal`` in that order from one
    generator seeded with the config's seed.
  * bf16 configs round each float32 value to bf16 with round-to-nearest-even
    (``round_to_bf16``); the oracle receives the same rounded values widened
    to float64, so both sides see identical inputs.
  * positions are 0..N-1 for prefill; decode puts the query at the cache length
    and the cache at 0..len-1.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


# ----------------------------------------------------------------------------
# bf16 helpers (pure bit manipulation, no attention arithmetic)
# ----------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the raw 16-bit patterns as ``uint16``.  Inputs here are finite
    normal draws, so no NaN handling is needed; a NaN would raise.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_to_bf16 expects finite values")
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = (bits + 0x7FFF + lsb) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) to float64: sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m * 2^-9); 0x7f / 0xff are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


_E4M3_GRID = e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))  # the 127 finite magnitudes, ascending


def round_to_e4m3(x: np.ndarray) -> np.ndarray:
    """float values to OCP FP8 E4M3 codes, round to nearest (ties to the even
    code), saturating at +-448.  Finite inputs only."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_to_e4m3 expects finite values")
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_GRID, a, side="left"), 0, 0x7E)  # first grid value >= a
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _E4M3_GRID[lo], _E4M3_GRID[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(x < 0, code | 0x80, code).astype(np.uint8)


# ----------------------------------------------------------------------------
# Workload descriptions
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "bf16" or "fp32"
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    D: int
    seed: int
    rope_theta: Optional[float] = None
    causal: bool = False
    window: int = 0
    alibi: bool = False
    bigbird_block: int = 0     # 0 = dense; else BigBird CSR with this block size
    q_pos0: int = 0
    k_pos0: int = 0
    decode_splits: int = 0     # >0: split-KV decode workload
    bias_heads: bool = False   # additive fp32 bias, one [Nq, Nk] plane per q-head (shared by batches)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads (sizes from the AttnFuse evaluation geometries).
WORKLOADS = {
    # fp32 RoPE+causal, small enough for the oracle to finish in well under 1 s.
    "rope_causal_fp32_n256": Workload(
        "rope_causal_fp32_n256", "fp32", B=1, Hq=4, Hkv=4, Nq=256, Nk=256, D=64,
        seed=1, rope_theta=10000.0, causal=True),
    # Llama-3-8B attention geometry, RoPE + causal prefill at N=4096.
    "llama3_8b_rope_causal_n4096": Workload(
        "llama3_8b_rope_causal_n4096", "bf16", B=1, Hq=32, Hkv=8, Nq=4096, Nk=4096,
        D=128, seed=2, rope_theta=500000.0, causal=True),
    # ALiBi + causal + sliding window W=1024, no RoPE.
    "alibi_causal_window1024_n8192": Workload(
        "alibi_causal_window1024_n8192", "bf16", B=2, Hq=16, Hkv=16, Nq=8192, Nk=8192,
        D=128, seed=3, causal=True, window=1024, alibi=True),
    # BigBird block-sparse (64x64 blocks) RoPE attention, non-causal.
    "bigbird_rope_n4096": Workload(
        "bigbird_rope_n4096", "bf16", B=2, Hq=16, Hkv=16, Nq=4096, Nk=4096, D=64,
        seed=4, rope_theta=10000.0, bigbird_block=64),
    # Llama-3-70B single-token decode over a 32k cache, 64 KV splits.
    "llama3_70b_decode_32k": Workload(
        "llama3_70b_decode_32k", "bf16", B=1, Hq=64, Hkv=8, Nq=1, Nk=32768, D=128,
        seed=5, rope_theta=500000.0, q_pos0=32768, k_pos0=0, decode_splits=64),
}

# Additive-bias workload (the pages' additive_bias combinator, no evaluation
# geometry given): a relative-position-style bias plane per head, B=2 H=16
# N=2048 D=128, causal, bias iid N(0,1) float32 drawn after Q, K, V.
WORKLOADS["bias_heads_causal_n2048"] = Workload(
    "bias_heads_causal_n2048", "bf16", B=2, Hq=16, Hkv=16, Nq=2048, Nk=2048, D=128, seed=7,
    causal=True, bias_heads=True)

# Second grid: the GPT-2-small geometry of the pages' head-to-head tables
# ("6.1 Forward Head-to-Head on Ampere", Table 6: Dense, Causal, SW W=256,
# Causal+ALiBi; "6.2 RoPE on Ampere", Table 7: RoPE + Dense / Causal / SW),
# B=4, H=12, D=64, N in {512, 1024, 2048, 4096}, in bf16 (the pages: fp16).
GPT2_VARIANTS = {
    "dense": dict(),
    "causal": dict(causal=True),
    "sw256": dict(window=256),
    "causal_alibi": dict(causal=True, alibi=True),
    "rope_dense": dict(rope_theta=10000.0),
    "rope_causal": dict(rope_theta=10000.0, causal=True),
    "rope_sw256": dict(rope_theta=10000.0, window=256),
}
GPT2_NS = (512, 1024, 2048, 4096)


def gpt2_small(variant: str, N: int) -> Workload:
    """GPT-2-small geometry workload (seed 6 for every cell)."""
    return Workload(f"gpt2s_{variant}_n{N}", "bf16", B=4, Hq=12, Hkv=12, Nq=N, Nk=N, D=64,
                    seed=6, **GPT2_VARIANTS[variant])


def alibi_slopes(H: int) -> np.ndarray:
    """ALiBi head slopes 2^(-8h/H) for h = 1..H, as float32 (index 0 = head 0)."""
    h = np.arange(1, H + 1, dtype=np.float64)
    return np.exp2(-8.0 * h / H).astype(np.float32)


def bigbird_csr(n_qblocks: int, n_kblocks: int, seed: int, n_window: int = 1,
                n_global: int = 2, n_random: int = 3):
    """BigBird-style block mask as CSR (row_ptr int32 [nqb+1], col_idx int32 [nnz]).

    Per query block ``qb`` the active key blocks are: the window
    ``qb-n_window .. qb+n_window`` clipped to range, the first ``n_global`` key
    blocks, and ``n_random`` further key blocks drawn without replacement from
    the blocks not already chosen (``numpy.random.default_rng(seed)``, rows in
    order).  Column lists are sorted.  One mask serves every (batch, head).
    """
    rng = np.random.default_rng(seed)
    row_ptr = [0]
    cols_all = []
    for qb in range(n_qblocks):
        chosen = set(range(max(0, qb - n_window), min(n_kblocks, qb + n_window + 1)))
        chosen |= set(range(min(n_global, n_kblocks)))
        rest = np.array(sorted(set(range(n_kblocks)) - chosen), dtype=np.int64)
        k = min(n_random, rest.size)
        if k:
            chosen |= set(int(c) for c in rng.choice(rest, size=k, replace=False))
        cols = sorted(chosen)
        cols_all.extend(cols)
        row_ptr.append(len(cols_all))
    return np.asarray(row_ptr, dtype=np.int32), np.asarray(cols_all, dtype=np.int32)


def random_csr(n_qblocks: int, n_kblocks: int, density: float, seed: int,
               n_heads: int = 0):
    """Random block mask (each block active with probability ``density``).

    With ``n_heads`` > 0 the result holds one CSR row set per head:
    row_ptr has shape [n_heads, nqb+1] with offsets into one shared col_idx.
    Rows may be empty (no active block).
    """
    rng = np.random.default_rng(seed)
    heads = max(1, n_heads)
    row_ptr = np.zeros((heads, n_qblocks + 1), dtype=np.int32)
    cols_all = []
    for h in range(heads):
        for qb in range(n_qblocks):
            row_ptr[h, qb] = len(cols_all)
            act = np.nonzero(rng.random(n_kblocks) < density)[0]
            cols_all.extend(int(c) for c in act)
        row_ptr[h, n_qblocks] = len(cols_all)
    col_idx = np.asarray(cols_all, dtype=np.int32)
    if n_heads == 0:
        return row_ptr[0], col_idx
    return row_ptr, col_idx


@dataclasses.dataclass
class Inputs:
    """Host copies of one workload's inputs.

    ``q``, ``k``, ``v`` are float64 arrays holding exactly the values the GPU
    receives; ``*_bits`` hold the bf16 patterns (bf16 workloads) and ``*_f32``
    the float32 values (fp32 workloads).
    """
    w: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_dev: np.ndarray       # uint16 bf16 bits or float32, laid out [B, H, N, D]
    k_dev: np.ndarray
    v_dev: np.ndarray
    alibi_slopes: Optional[np.ndarray] = None
    bias: Optional[np.ndarray] = None   # float32 [1, Hq, Nq, Nk] (broadcast over batches)
    bs_row_ptr: Optional[np.ndarray] = None
    bs_col_idx: Optional[np.ndarray] = None


def make_inputs(w: Workload, seed: Optional[int] = None) -> Inputs:
    rng = np.random.default_rng(w.seed if seed is None else seed)
    qs = (w.B, w.Hq, w.Nq, w.D)
    ks = (w.B, w.Hkv, w.Nk, w.D)
    q32 = rng.standard_normal(qs, dtype=np.float32)
    k32 = rng.standard_normal(ks, dtype=np.float32)
    v32 = rng.standard_normal(ks, dtype=np.float32)
    if w.dtype == "bf16":
        qb, kb, vb = round_to_bf16(q32), round_to_bf16(k32), round_to_bf16(v32)
        inp = Inputs(w, bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb),
                     qb, kb, vb)
    elif w.dtype == "fp32":
        inp = Inputs(w, q32.astype(np.float64), k32.astype(np.float64),
                     v32.astype(np.float64), q32, k32, v32)
    else:
        raise ValueError(w.dtype)
    if w.alibi:
        inp.alibi_slopes = alibi_slopes(w.Hq)
    if w.bias_heads:
        inp.bias = rng.standard_normal((1, w.Hq, w.Nq, w.Nk), dtype=np.float32)
    if w.bigbird_block:
        nqb = -(-w.Nq // w.bigbird_block)
        nkb = -(-w.Nk // w.bigbird_block)
        inp.bs_row_ptr, inp.bs_col_idx = bigbird_csr(nqb, nkb, seed=w.seed)
    return inp


def normal_e4m3(shape, rng: np.random.Generator):
    """N(0,1) float32 draws quantised to OCP E4M3 with a per-tensor scale
    (largest magnitude -> 448): (codes uint8, dequantised float64 values
    code * scale, scale)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    scale = float(np.abs(x).max()) / 448.0
    codes = round_to_e4m3(x / scale)
    return codes, e4m3_to_f64(codes) * scale, scale


def normal_bf16(shape, rng: np.random.Generator, scale: float = 1.0):
    """(bits uint16, float64 values) of scaled N(0,1) draws rounded to bf16."""
    x = (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)
    bits = round_to_bf16(x)
    return bits, bf16_bits_to_f64(bits)
