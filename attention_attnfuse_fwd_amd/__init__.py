"""MI355X (gfx950) fused attention forward: RoPE, causal / sliding-window /
block-sparse masks, ALiBi and additive bias composed into one HIP kernel, plus
a split-KV decode with a log-sum-exp combine, and the attention backward.

The compute lives in ``libattnfuse.so`` (C ABI in ``include/attnfuse.h``);
this package only marshals PyTorch tensors and streams into it.
"""
from ._abi import LIB_PATH, LibraryNotBuilt, VariantDesc, library_identity, load as load_library  # noqa: F401
from .ops import (AttnfuseError, BlockMask, block_mask_from_csr, bwd, bwd_workspace_size,  # noqa: F401
                  bigbird_block_mask, create_block_mask,
                  decode, decode_noalloc, decode_workspace_size, default_num_splits, fwd, fwd_plan,
                  prerotate,
                  rope_tables)

__all__ = [
    "fwd", "fwd_plan", "bwd", "bwd_workspace_size", "decode", "decode_noalloc", "decode_workspace_size", "default_num_splits", "prerotate",
    "rope_tables", "create_block_mask", "bigbird_block_mask", "block_mask_from_csr", "BlockMask", "AttnfuseError",
    "load_library", "library_identity", "LIB_PATH", "LibraryNotBuilt", "VariantDesc",
]
