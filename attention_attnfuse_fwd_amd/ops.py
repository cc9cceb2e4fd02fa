"""PyTorch-facing entry points over the C ABI (argument marshalling only).

Every step of the computation runs in the HIP kernels of ``libattnfuse.so``;
PyTorch supplies device memory and the current HIP stream.  Names follow the
AttnFuse pages ("AttnFuse: A Composable DSL for Compiling Attentions to Fused
GPU Kernels"): ``fwd`` is the fused forward of "3.3 Runtime Dispatch" with its
decode fast path, ``decode`` the split-KV path of "4.2 Flash Decoding",
``create_block_mask`` builds the CSR BlockMask of "4.3 Block-Sparse
Attention" and ``bigbird_block_mask`` its BigBird instance, ``rope_tables``
the precomputed cos / sin tables of "4.1 Fused RoPE", and ``prerotate`` the
separate rotation pass that fusion replaces.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Callable, Optional

import numpy as np
import torch

from . import _abi


class AttnfuseError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"attnfuse error {status} ({_abi.status_string(status)}){': ' + what if what else ''}")


def _check(status: int, what: str = ""):
    if status != _abi.OK:
        raise AttnfuseError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _raw_stream(device: torch.device) -> int:
    """Handle of the current stream of ``device`` as an int."""
    if _RAW_STREAM is not None:
        return _RAW_STREAM(device.index)
    return torch.cuda.current_stream(device).cuda_stream


# Prepared descriptors of calls whose descriptor holds no per-call pointer
# (no lse output, ALiBi slopes, bias or block mask): keyed by everything the
# descriptor is built from, so a repeated call skips the marshalling.  A
# cached descriptor is never modified after it is stored.
_FWD_DESCS: dict = {}
_DECODE_DESCS: dict = {}


_E4M3 = getattr(torch, "float8_e4m3fn", None)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16 or (_E4M3 is not None and t.dtype == _E4M3):
        return _abi.BF16  # fp8 inputs produce a bf16 output
    if t.dtype == torch.float32:
        return _abi.FP32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16, float32 or float8_e4m3fn")


# ----------------------------------------------------------------------------
# RoPE tables
# ----------------------------------------------------------------------------

class _RopeEntry:
    """One cached table set: fp32 cos, fp32 sin and packed fp16 (cos, sin)
    words, built asynchronously on ``stream``; ``ready`` marks the end of the
    build on that stream."""
    __slots__ = ("cos", "sin", "cs16", "ready", "stream", "done")

    def __init__(self, cos, sin, cs16, ready, stream):
        self.cos, self.sin, self.cs16 = cos, sin, cs16
        self.ready, self.stream, self.done = ready, stream, False


_ROPE_CACHE: dict = {}
# Tables replaced by longer ones stay alive until the process ends: kernels
# already queued on any stream may still read them.
_ROPE_RETIRED: list = []


def _rope_entry(theta: float, D: int, length: int, device: torch.device) -> _RopeEntry:
    index = device.index if device.index is not None else torch.cuda.current_device()
    key = (float(theta), int(D), index)
    hit = _ROPE_CACHE.get(key)
    if hit is not None and hit.cos.shape[0] >= length:
        return hit
    L = max(int(length), 1)
    if hit is not None:
        L = max(L, 2 * hit.cos.shape[0])
        _ROPE_RETIRED.append(hit)
    cos = torch.empty((L, D // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    cs16 = torch.empty((L, D // 2), dtype=torch.int32, device=device)
    stream = torch.cuda.current_stream(device)
    _check(_abi.load().attnfuse_rope_table(float(theta), int(D), int(L), _ptr(cos), _ptr(sin),
                                           _ptr(cs16), None, ctypes.c_void_p(stream.cuda_stream)),
           "rope_table")
    ready = torch.cuda.Event()
    ready.record(stream)
    entry = _RopeEntry(cos, sin, cs16, ready, stream.cuda_stream)
    _ROPE_CACHE[key] = entry
    return entry


def _rope_ready_on(entry: _RopeEntry, device: torch.device):
    """Order the current stream after the table's build (once the build is
    known to be complete, no further waits are issued)."""
    if entry.done:
        return
    if entry.ready.query():
        entry.done = True
        return
    cur = torch.cuda.current_stream(device)
    if cur.cuda_stream != entry.stream:
        cur.wait_event(entry.ready)


def rope_tables(theta: float, D: int, length: int, device) -> tuple:
    """(cos, sin, cs_f16) tables [L][D/2] with L >= length, built on the device
    and cached per (theta, D, device): fp32 cos and sin (fp32 kernels, the
    pre-rotation pass) and the packed fp16 (cos, sin) words the bf16 kernels
    read.  The current stream is ordered after the build."""
    device = torch.device(device)
    entry = _rope_entry(theta, D, length, device)
    _rope_ready_on(entry, device)
    return entry.cos, entry.sin, entry.cs16


# ----------------------------------------------------------------------------
# Block masks
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class BlockMask:
    """CSR block mask: per query block, the list of active key blocks."""
    row_ptr: torch.Tensor        # int32 [nqb + 1] (shared) or [H, nqb + 1] (per q-head)
    col_idx: torch.Tensor        # int32 [nnz]
    block_m: int
    block_n: int

    @property
    def nnz(self) -> int:
        return int(self.col_idx.numel())

    @property
    def per_head(self) -> bool:
        return self.row_ptr.dim() == 2


def block_mask_from_csr(row_ptr, col_idx, block_m: int, block_n: int, device) -> BlockMask:
    rp = torch.as_tensor(np.asarray(row_ptr, dtype=np.int32)).to(device)
    ci = torch.as_tensor(np.asarray(col_idx, dtype=np.int32)).to(device)
    if ci.numel() == 0:
        ci = torch.zeros(1, dtype=torch.int32, device=device)[:0]
    return BlockMask(rp.contiguous(), ci.contiguous(), int(block_m), int(block_n))


def create_block_mask(predicate: Callable, n_qblocks: int, n_kblocks: int, block_m: int,
                      block_n: int, device, heads: Optional[int] = None) -> BlockMask:
    """Evaluate ``predicate(qb, kb)`` (or ``predicate(h, qb, kb)`` with ``heads``)
    once for every block pair on the host and return the CSR BlockMask."""
    rows = []
    cols = []
    for h in range(heads or 1):
        rp = [len(cols)]
        for qb in range(n_qblocks):
            for kb in range(n_kblocks):
                ok = predicate(h, qb, kb) if heads else predicate(qb, kb)
                if ok:
                    cols.append(kb)
            rp.append(len(cols))
        rows.append(rp)
    row_ptr = np.asarray(rows if heads else rows[0], dtype=np.int32)
    return block_mask_from_csr(row_ptr, np.asarray(cols, dtype=np.int32), block_m, block_n, device)


def bigbird_block_mask(N: int, block: int, n_window: int = 1, n_global: int = 2,
                       n_random: int = 3, seed: int = 0, device="cpu",
                       N_k: Optional[int] = None) -> BlockMask:
    """BigBird block mask ("4.3 Block-Sparse Attention", BigBird reference [9]).

    Square ``block`` x ``block`` tiles over ``N`` queries and ``N_k`` keys
    (default ``N``).  Query block ``i`` attends to the key blocks of its
    neighbourhood ``i - n_window .. i + n_window`` (clipped), to the first
    ``n_global`` key blocks, and to ``n_random`` more key blocks drawn without
    replacement from the ones not already active, with
    ``numpy.random.default_rng(seed)`` consumed query block by query block in
    increasing order.  Each row's key blocks are stored in increasing order.
    The mask is shared by every batch and head; tail blocks of ragged ``N``
    are whole blocks (the kernel masks the positions past the end).
    """
    if N < 0 or block <= 0 or min(n_window, n_global, n_random) < 0:
        raise ValueError("bigbird_block_mask: N >= 0, block > 0 and non-negative counts required")
    nk = N if N_k is None else N_k
    nqb = -(-N // block)
    nkb = -(-nk // block)
    rng = np.random.default_rng(seed)
    row_ptr = np.zeros(nqb + 1, dtype=np.int32)
    cols = []
    for i in range(nqb):
        active = np.zeros(nkb, dtype=bool)
        active[max(0, i - n_window):min(nkb, i + n_window + 1)] = True
        active[:min(n_global, nkb)] = True
        free = np.flatnonzero(~active)
        take = min(n_random, free.size)
        if take:
            active[rng.choice(free, size=take, replace=False)] = True
        row = np.flatnonzero(active)
        cols.append(row)
        row_ptr[i + 1] = row_ptr[i] + row.size
    col_idx = np.concatenate(cols).astype(np.int32) if cols else np.zeros(0, dtype=np.int32)
    return block_mask_from_csr(row_ptr, col_idx, block, block, device)


# ----------------------------------------------------------------------------
# Descriptor marshalling
# ----------------------------------------------------------------------------

def _strides3(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, H, N, D]")
    if t.numel() == 0:  # nothing is read or written: describe it as contiguous
        _, H, N, D = t.shape
        return (H * N * D, N * D, D)
    if t.stride(3) != 1:
        raise ValueError(f"{name} must have a contiguous last (head) dimension")
    return (t.stride(0), t.stride(1), t.stride(2))


def _make_desc(q, k, v, out, *, scale, causal, window, rope_theta, q_pos0, k_pos0,
               alibi_slopes, bias, block_mask, lse, keep):
    d = _abi.VariantDesc.new()
    d.dtype = _dtype_code(q)
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = k.shape
    d.B, d.Hq, d.Hkv, d.Nq, d.Nk, d.D = B, Hq, Hkv, Nq, Nk, D
    for name, t, field in (("q", q, "q_stride"), ("k", k, "k_stride"), ("v", v, "v_stride"),
                           ("out", out, "o_stride")):
        s = _strides3(t, name)
        arr = getattr(d, field)
        arr[0], arr[1], arr[2] = s
    d.scale = 0.0 if scale is None else float(scale)
    d.norm = _abi.NORM_SOFTMAX
    d.q_pos0, d.k_pos0 = int(q_pos0), int(k_pos0)
    d.causal = 1 if causal else 0
    d.window = int(window or 0)
    if rope_theta is not None:
        need = max(int(q_pos0) + Nq, int(k_pos0) + Nk)
        cos, sin, cs16 = rope_tables(rope_theta, D, need, q.device)
        keep.extend([cos, sin, cs16])
        d.rope = 1
        d.rope_theta = float(rope_theta)
        d.rope_cos, d.rope_sin = cos.data_ptr(), sin.data_ptr()
        d.rope_cs_f16 = cs16.data_ptr()
        d.rope_table_len = cos.shape[0]
    if alibi_slopes is not None:
        a = torch.as_tensor(alibi_slopes, dtype=torch.float32).to(q.device).contiguous()
        if a.numel() != Hq:
            raise ValueError("alibi_slopes needs one slope per query head")
        keep.append(a)
        d.alibi_slopes = a.data_ptr()
    if bias is not None:
        bt = torch.as_tensor(bias).to(device=q.device, dtype=torch.float32)
        if bt.dim() != 4:
            raise ValueError("bias must be 4-D, broadcastable to [B, Hq, Nq, Nk]")
        bt = bt.expand(B, Hq, Nq, Nk)
        keep.append(bt)
        d.bias = bt.data_ptr()
        for a in range(4):
            d.bias_stride[a] = bt.stride(a)
    if block_mask is not None:
        keep.extend([block_mask.row_ptr, block_mask.col_idx])
        d.bs_row_ptr = block_mask.row_ptr.data_ptr()
        d.bs_col_idx = block_mask.col_idx.data_ptr() if block_mask.nnz else None
        d.bs_block_m, d.bs_block_n = block_mask.block_m, block_mask.block_n
        d.bs_head_stride = block_mask.row_ptr.shape[1] if block_mask.per_head else 0
        d.bs_nnz = block_mask.nnz
    if lse is not None:
        d.lse = lse.data_ptr()
    return d


def _set_tile(d, tile):
    """``tile = (waves, heads)`` or ``(waves, heads, chain)``; 0 = the library's choice."""
    d.tile_waves, d.tile_heads = int(tile[0]), int(tile[1])
    if len(tile) > 2:
        d.tile_chain = int(tile[2])


def _check_inputs(q, k, v):
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")


def default_num_splits(B: int, Hkv: int, G: int, Nk: int, target_wgs: int = 512) -> int:
    """Split count that gives the decode phase 1 about ``target_wgs`` workgroups."""
    units = B * Hkv * ((G + 31) // 32)
    s = max(1, round(target_wgs / max(units, 1)))
    return int(max(1, min(s, max(1, math.ceil(Nk / 128)), 4096)))


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
        window: int = 0, rope_theta: Optional[float] = None, q_pos0: int = 0, k_pos0: int = 0,
        alibi_slopes=None, bias=None, block_mask: Optional[BlockMask] = None,
        scale: Optional[float] = None, return_lse: bool = False,
        out: Optional[torch.Tensor] = None, decode_fast_path: bool = True,
        tile: Optional[tuple] = None, q_scale: float = 1.0, k_scale: float = 1.0,
        v_scale: float = 1.0):
    """Fused attention forward; q [B, Hq, Nq, D], k / v [B, Hkv, Nk, D] on the GPU.

    A single query row (Nq == 1, bf16, no bias or block mask) takes the split-KV
    decode path, as the pages' runtime dispatch does.  ``tile = (waves, heads)``
    or ``(waves, heads, chain)`` overrides the library's tile table for the
    bf16 prefill kernel (0 = the library's choice; ``chain``: query blocks per
    workgroup of a block-sparse launch on two or four waves).  With
    ``torch.float8_e4m3fn`` q, k and v (E4M3 codes whose rows are
    ``q_scale * code`` etc.) the fp8 prefill runs and the output is bf16.
    """
    cacheable = (out is not None and not return_lse and alibi_slopes is None and bias is None
                 and block_mask is None)
    if cacheable:
        key = (q.shape, q.stride(), k.shape, k.stride(), v.shape, v.stride(), out.shape, out.stride(),
               q.dtype, k.dtype, v.dtype, out.dtype, q.device, k.device, v.device, out.device,
               causal, window, rope_theta, q_pos0, k_pos0, scale, decode_fast_path, q_scale, k_scale,
               v_scale, None if tile is None else tuple(int(x) for x in tile))
        hit = _FWD_DESCS.get(key)
        if hit is not None:
            dref, entry = hit
            if entry is not None:
                _rope_ready_on(entry, q.device)
            _check(_abi.load().attnfuse_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                            dref, _raw_stream(q.device)), "fwd")
            return out
    _check_inputs(q, k, v)
    if (decode_fast_path and q.shape[2] == 1 and q.dtype == torch.bfloat16 and bias is None
            and block_mask is None and k.shape[2] > 0):
        return decode(q, k, v, causal=causal, window=window, rope_theta=rope_theta,
                      q_pos0=q_pos0, k_pos0=k_pos0, alibi_slopes=alibi_slopes, scale=scale,
                      return_lse=return_lse, out=out)
    fp8 = _E4M3 is not None and q.dtype == _E4M3
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16 if fp8 else q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    keep = []
    d = _make_desc(q, k, v, out, scale=scale, causal=causal, window=window,
                   rope_theta=rope_theta, q_pos0=q_pos0, k_pos0=k_pos0,
                   alibi_slopes=alibi_slopes, bias=bias, block_mask=block_mask, lse=lse,
                   keep=keep)
    if fp8:
        d.kv_fp8, d.q_fp8 = 1, 1
        d.q_scale, d.k_scale, d.v_scale = float(q_scale), float(k_scale), float(v_scale)
    if tile is not None:
        _set_tile(d, tile)
    _check(_abi.load().attnfuse_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), ctypes.byref(d),
                                    _stream(q.device)), "fwd")
    if cacheable:
        entry = (_ROPE_CACHE.get((float(rope_theta), int(q.shape[3]), q.device.index))
                 if rope_theta is not None else None)
        if entry is None or entry.cos.data_ptr() == d.rope_cos:
            _FWD_DESCS[key] = (ctypes.byref(d), entry)
    return (out, lse) if return_lse else out


def fwd_plan(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
             window: int = 0, rope_theta: Optional[float] = None, q_pos0: int = 0, k_pos0: int = 0,
             alibi_slopes=None, bias=None, block_mask: Optional[BlockMask] = None,
             scale: Optional[float] = None, tile: Optional[tuple] = None) -> dict:
    """The launch ``fwd`` would make for these arguments (prefill kernels; the
    single-query decode path is not considered): kernel, waves and q-heads per
    workgroup, query rows per block, blocks per unit, pairing, grid and
    block-sparse chain length."""
    _check_inputs(q, k, v)
    keep = []
    d = _make_desc(q, k, v, q, scale=scale, causal=causal, window=window, rope_theta=rope_theta,
                   q_pos0=q_pos0, k_pos0=k_pos0, alibi_slopes=alibi_slopes, bias=bias,
                   block_mask=block_mask, lse=None, keep=keep)
    if _E4M3 is not None and q.dtype == _E4M3:
        d.kv_fp8, d.q_fp8 = 1, 1
        d.q_scale = d.k_scale = d.v_scale = 1.0  # (scales do not change the launch)
    if tile is not None:
        _set_tile(d, tile)
    info = _abi.FwdPlanInfo()
    _check(_abi.load().attnfuse_fwd_plan(ctypes.byref(d), ctypes.byref(info)), "fwd_plan")
    out = {f: getattr(info, f) for f, _ in _abi.FwdPlanInfo._fields_}
    out["kernel"] = _abi.PLAN_KERNELS[info.kernel]
    return out


def decode_workspace_size(q, k_cache, num_splits: int) -> int:
    d = _abi.VariantDesc.new()
    d.dtype = _dtype_code(q)
    d.B, d.Hq, d.Nq, d.D = q.shape
    d.Hkv, d.Nk = k_cache.shape[1], k_cache.shape[2]
    for f, t in (("q_stride", q), ("k_stride", k_cache), ("v_stride", k_cache), ("o_stride", q)):
        arr = getattr(d, f)
        arr[0], arr[1], arr[2] = _strides3(t, f)
    return int(_abi.load().attnfuse_decode_workspace_size(ctypes.byref(d), int(num_splits)))


_FP8_DTYPES = tuple(t for t in (getattr(torch, "float8_e4m3fn", None), torch.uint8) if t is not None)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, *,
           num_splits: Optional[int] = None, causal: bool = False, window: int = 0,
           rope_theta: Optional[float] = None, q_pos0: int = 0, k_pos0: int = 0,
           alibi_slopes=None, scale: Optional[float] = None, return_lse: bool = False,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           k_scale: float = 1.0, v_scale: float = 1.0):
    """Split-KV single-query decode (q [B, Hq, 1, D] bf16) with a log-sum-exp combine.

    The cache is bf16 like q, or FP8 E4M3 codes (``torch.float8_e4m3fn``, or
    their bytes as ``torch.uint8``) holding rows ``k_scale * code`` and
    ``v_scale * code``."""
    cacheable = (out is not None and workspace is not None and not return_lse and alibi_slopes is None
                 and num_splits is not None)
    if cacheable:
        key = (q.shape, q.stride(), k_cache.shape, k_cache.stride(), v_cache.shape, v_cache.stride(),
               out.shape, out.stride(), q.dtype, k_cache.dtype, v_cache.dtype, out.dtype, q.device,
               k_cache.device, v_cache.device, out.device, num_splits, causal, window, rope_theta,
               q_pos0, k_pos0, scale, k_scale, v_scale, workspace.device)
        hit = _DECODE_DESCS.get(key)
        nbytes = workspace.numel() * workspace.element_size()
        if hit is not None and nbytes >= hit[2]:
            dref, entry, _ = hit
            if entry is not None:
                _rope_ready_on(entry, q.device)
            _check(_abi.load().attnfuse_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                               out.data_ptr(), dref, int(num_splits), workspace.data_ptr(),
                                               nbytes, _raw_stream(q.device)), "decode")
            return out
    kv_fp8 = k_cache.dtype in _FP8_DTYPES
    if kv_fp8:
        if v_cache.dtype != k_cache.dtype or q.dtype != torch.bfloat16:
            raise TypeError("an fp8 cache needs fp8 k_cache and v_cache and a bf16 query")
        if not (q.is_cuda and k_cache.is_cuda and v_cache.is_cuda):
            raise ValueError("q, k_cache, v_cache must be GPU tensors")
        if k_cache.shape != v_cache.shape:
            raise ValueError("k and v must have the same shape")
    else:
        _check_inputs(q, k_cache, v_cache)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    if num_splits is None:
        num_splits = default_num_splits(B, Hkv, Hq // max(Hkv, 1), Nk)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if return_lse else None
    keep = []
    d = _make_desc(q, k_cache, v_cache, out, scale=scale, causal=causal, window=window,
                   rope_theta=rope_theta, q_pos0=q_pos0, k_pos0=k_pos0,
                   alibi_slopes=alibi_slopes, bias=None, block_mask=None, lse=lse, keep=keep)
    if kv_fp8:
        d.kv_fp8, d.k_scale, d.v_scale = 1, float(k_scale), float(v_scale)
    lib = _abi.load()
    need = int(lib.attnfuse_decode_workspace_size(ctypes.byref(d), int(num_splits)))
    if workspace is None:
        workspace = torch.empty(max(need, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.attnfuse_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), ctypes.byref(d),
                               int(num_splits), _ptr(workspace), nbytes, _stream(q.device)),
           "decode")
    if cacheable:
        entry = (_ROPE_CACHE.get((float(rope_theta), int(D), q.device.index))
                 if rope_theta is not None else None)
        if entry is None or entry.cos.data_ptr() == d.rope_cos:
            _DECODE_DESCS[key] = (ctypes.byref(d), entry, need)
    return (out, lse) if return_lse else out


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, out: torch.Tensor, *,
                   num_splits: int, causal: bool = False, window: int = 0,
                   rope_theta: Optional[float] = None, q_pos0: int = 0, k_pos0: int = 0,
                   alibi_slopes: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                   lse: Optional[torch.Tensor] = None, k_scale: float = 1.0, v_scale: float = 1.0):
    """``decode`` without a workspace (``attnfuse_decode_noalloc``): the
    partials go to the library's static per-GPU buffer, so neither this call
    nor the library allocates device memory (``out``, and ``lse`` [B, Hq, 1]
    fp32 when wanted, are the caller's; the RoPE table must already be built,
    e.g. by ``rope_tables``, or it is built and cached on first use).  Calls
    that may overlap on one GPU race on that buffer.  Returns ``out``."""
    kv_fp8 = k_cache.dtype in _FP8_DTYPES
    if not kv_fp8:
        _check_inputs(q, k_cache, v_cache)
    elif not (q.is_cuda and k_cache.is_cuda and v_cache.is_cuda) or k_cache.shape != v_cache.shape:
        raise ValueError("q, k_cache, v_cache must be GPU tensors, k and v of one shape")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != q.shape[:3] or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, Hq, 1] tensor")
    keep = []
    d = _make_desc(q, k_cache, v_cache, out, scale=scale, causal=causal, window=window,
                   rope_theta=rope_theta, q_pos0=q_pos0, k_pos0=k_pos0, alibi_slopes=alibi_slopes,
                   bias=None, block_mask=None, lse=lse, keep=keep)
    if kv_fp8:
        d.kv_fp8, d.k_scale, d.v_scale = 1, float(k_scale), float(v_scale)
    _check(_abi.load().attnfuse_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                               ctypes.byref(d), int(num_splits), _stream(q.device)),
           "decode_noalloc")
    return out


def bwd_workspace_size(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                       window: int = 0, rope_theta: Optional[float] = None, q_pos0: int = 0,
                       k_pos0: int = 0) -> int:
    """Bytes of workspace bwd() needs for these shapes and masks (the row
    reductions, the rotated Q and K when rope_theta is given, and fp32
    partial dK / dV sums when a band's key blocks are split)."""
    _check_inputs(q, k, v)
    keep = []
    d = _make_desc(q, k, v, q, scale=None, causal=causal, window=window, rope_theta=rope_theta,
                   q_pos0=q_pos0, k_pos0=k_pos0, alibi_slopes=None, bias=None, block_mask=None,
                   lse=None, keep=keep)
    return int(_abi.load().attnfuse_bwd_workspace_size(ctypes.byref(d)))


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
        lse: torch.Tensor, *, causal: bool = False, window: int = 0,
        rope_theta: Optional[float] = None, q_pos0: int = 0, k_pos0: int = 0,
        alibi_slopes=None, bias=None, block_mask: Optional[BlockMask] = None,
        scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None):
    """Attention backward ("4.4 Backward Pass"): returns (dq, dk, dv), the
    gradients of sum(out * dout) for the forward fwd(q, k, v, ...) computed
    with the same keyword arguments; ``out`` and ``lse`` are that forward's
    output and saved statistic (``fwd(..., return_lse=True)``).  bf16; an
    additive bias is a constant of the forward (no bias gradient); a block
    mask restricts both gradient passes to the listed blocks.  dq / dk / dv
    have the strides of q / k / v."""
    _check_inputs(q, k, v)
    if dout.shape != out.shape:
        raise ValueError("dout must have the shape of out")
    if dout.stride() != out.stride():
        dout = torch.empty_like(out).copy_(dout)
    if lse.shape != q.shape[:3] or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hq, Nq]")
    lse = lse.contiguous()
    dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
    dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=v.device)
    keep = []
    d = _make_desc(q, k, v, out, scale=scale, causal=causal, window=window,
                   rope_theta=rope_theta, q_pos0=q_pos0, k_pos0=k_pos0,
                   alibi_slopes=alibi_slopes, bias=bias, block_mask=block_mask, lse=None,
                   keep=keep)
    lib = _abi.load()
    need = int(lib.attnfuse_bwd_workspace_size(ctypes.byref(d)))
    if workspace is None:
        workspace = torch.empty(max(need, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.attnfuse_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq),
                            _ptr(dk), _ptr(dv), ctypes.byref(d), _ptr(workspace), nbytes,
                            _stream(q.device)), "bwd")
    return dq, dk, dv


def prerotate(x: torch.Tensor, *, rope_theta: float, pos0: int = 0, out: Optional[torch.Tensor] = None):
    """RoPE(x) into a new tensor (the separate pre-rotation pass)."""
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    if out is None:
        out = torch.empty_like(x)
    if out.stride() != x.stride():
        raise ValueError("out must have the same strides as x")
    keep = []
    # Describe x as the key tensor (which = 1) of a one-query problem.
    qdummy = x[:, :1, :1]
    d = _make_desc(qdummy, x, x, qdummy, scale=None, causal=False, window=0,
                   rope_theta=rope_theta, q_pos0=0, k_pos0=pos0, alibi_slopes=None, bias=None,
                   block_mask=None, lse=None, keep=keep)
    d.Hq = d.Hkv = x.shape[1]
    _check(_abi.load().attnfuse_prerotate(_ptr(x), _ptr(out), ctypes.byref(d), 1, _stream(x.device)),
           "prerotate")
    return out
