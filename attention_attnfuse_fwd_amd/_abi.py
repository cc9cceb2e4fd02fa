"""ctypes view of the C ABI declared in ``include/attnfuse.h``.

Loads ``libattnfuse.so`` from this package directory.  There is no fallback:
if the library is missing, loading raises ``LibraryNotBuilt``.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattnfuse.so")

OK = 0
ERR_INVALID = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE = -3
ERR_HIP = -4

# attnfuse_decode_noalloc's static partials buffer (ATTNFUSE_DECODE_NOALLOC_MAX_BYTES)
DECODE_NOALLOC_MAX_BYTES = 8 << 20

BF16 = 0
FP32 = 1
NORM_SOFTMAX = 0
NORM_RELU = 1

# Every function the headers declare (checked against include/*.h by the tests).
EXPORTS = (
    "attnfuse_fwd",
    "attnfuse_fwd_plan",
    "attnfuse_decode_workspace_size",
    "attnfuse_decode",
    "attnfuse_decode_noalloc",
    "attnfuse_rope_table",
    "attnfuse_prerotate",
    "attnfuse_bwd_workspace_size",
    "attnfuse_bwd",
    "attnfuse_status_string",
    # include/attnfuse_microbench.h
    "attnfuse_mb_mfma_bf16",
    "attnfuse_mb_mfma_bf16_ops",
    "attnfuse_mb_hbm_read",
    "attnfuse_mb_host_cost",
)


PLAN_KERNELS = {0: "none", 1: "fp32", 2: "bf16", 3: "fp8"}


class FwdPlanInfo(ctypes.Structure):
    """Mirror of ``attnfuse_fwd_plan_info``."""
    _fields_ = [
        ("kernel", ctypes.c_int32),
        ("waves", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("rows", ctypes.c_int32),
        ("query_blocks", ctypes.c_int32),
        ("paired", ctypes.c_int32),
        ("workgroups", ctypes.c_int64),
        ("chain", ctypes.c_int32),
    ]


class LibraryNotBuilt(ImportError):
    pass


class VariantDesc(ctypes.Structure):
    """Mirror of ``attnfuse_variant_desc`` (field order and types as in the header)."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32),
        ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("Nq", ctypes.c_int32),
        ("Nk", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3),
        ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
        ("scale", ctypes.c_float),
        ("norm", ctypes.c_int32),
        ("rope", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("rope_cos", ctypes.c_void_p),
        ("rope_sin", ctypes.c_void_p),
        ("rope_cs_f16", ctypes.c_void_p),
        ("rope_cs_bf16", ctypes.c_void_p),
        ("rope_table_len", ctypes.c_int64),
        ("q_pos0", ctypes.c_int64),
        ("k_pos0", ctypes.c_int64),
        ("causal", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("alibi_slopes", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("bias_stride", ctypes.c_int64 * 4),
        ("bs_row_ptr", ctypes.c_void_p),
        ("bs_col_idx", ctypes.c_void_p),
        ("bs_block_m", ctypes.c_int32),
        ("bs_block_n", ctypes.c_int32),
        ("bs_head_stride", ctypes.c_int64),
        ("bs_nnz", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("tile_waves", ctypes.c_int32),
        ("tile_heads", ctypes.c_int32),
        ("kv_fp8", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("q_fp8", ctypes.c_int32),
        ("q_scale", ctypes.c_float),
        ("tile_chain", ctypes.c_int32),
    ]

    @classmethod
    def new(cls) -> "VariantDesc":
        d = cls()
        d.struct_size = ctypes.sizeof(cls)
        return d


_lib = None


def load() -> ctypes.CDLL:
    """Load the library once and declare argument / return types."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryNotBuilt(
            f"{LIB_PATH} is missing; build it with `python -m attention_attnfuse_fwd_amd.build` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(VariantDesc)
    lib.attnfuse_fwd.argtypes = [P, P, P, P, D, P]
    lib.attnfuse_fwd.restype = ctypes.c_int
    lib.attnfuse_fwd_plan.argtypes = [D, ctypes.POINTER(FwdPlanInfo)]
    lib.attnfuse_fwd_plan.restype = ctypes.c_int
    lib.attnfuse_decode_workspace_size.argtypes = [D, ctypes.c_int32]
    lib.attnfuse_decode_workspace_size.restype = ctypes.c_size_t
    lib.attnfuse_decode.argtypes = [P, P, P, P, D, ctypes.c_int32, P, ctypes.c_size_t, P]
    lib.attnfuse_decode.restype = ctypes.c_int
    lib.attnfuse_decode_noalloc.argtypes = [P, P, P, P, D, ctypes.c_int32, P]
    lib.attnfuse_decode_noalloc.restype = ctypes.c_int
    lib.attnfuse_rope_table.argtypes = [ctypes.c_double, ctypes.c_int32, ctypes.c_int64, P, P, P, P, P]
    lib.attnfuse_rope_table.restype = ctypes.c_int
    lib.attnfuse_prerotate.argtypes = [P, P, D, ctypes.c_int32, P]
    lib.attnfuse_prerotate.restype = ctypes.c_int
    lib.attnfuse_bwd_workspace_size.argtypes = [D]
    lib.attnfuse_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attnfuse_bwd.argtypes = [P, P, P, P, P, P, P, P, P, D, P, ctypes.c_size_t, P]
    lib.attnfuse_bwd.restype = ctypes.c_int
    lib.attnfuse_status_string.argtypes = [ctypes.c_int]
    lib.attnfuse_status_string.restype = ctypes.c_char_p
    lib.attnfuse_mb_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, P]
    lib.attnfuse_mb_mfma_bf16.restype = ctypes.c_int
    lib.attnfuse_mb_mfma_bf16_ops.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, P, P]
    lib.attnfuse_mb_mfma_bf16_ops.restype = ctypes.c_int
    lib.attnfuse_mb_hbm_read.argtypes = [P, ctypes.c_size_t, ctypes.c_int32, P, P, P]
    lib.attnfuse_mb_hbm_read.restype = ctypes.c_int
    lib.attnfuse_mb_host_cost.argtypes = [ctypes.c_int32, P, P, P, P, D, ctypes.c_int32, P, ctypes.c_size_t,
                                          ctypes.c_int32, ctypes.POINTER(ctypes.c_double), P]
    lib.attnfuse_mb_host_cost.restype = ctypes.c_int
    _lib = lib
    return lib


def library_identity() -> dict:
    """Path and sha256 of the library file this process loads."""
    import hashlib
    h = hashlib.sha256()
    with open(LIB_PATH, "rb") as fh:
        for chunk in iter(lambda: fh.read(1 << 20), b""):
            h.update(chunk)
    return {"path": os.path.relpath(LIB_PATH, os.path.dirname(os.path.dirname(LIB_PATH))),
            "sha256": h.hexdigest()}


def status_string(status: int) -> str:
    return load().attnfuse_status_string(status).decode()
