"""Paged KV-cache attention (decode and extend) for AMD Instinct MI355X (gfx950).

The kernels and the C ABI live in ``libpkv.so`` (sources in ``csrc/``, header
``include/pkv.h`` at the repository root); ``ops`` wraps them for torch
tensors.  Nothing here computes on the host: if the library is missing the
calls raise.
"""

from ._lib import PkvError, lib, LIB_PATH
from .ops import (
    cache_desc,
    decode_partition_tokens,
    decode_runs,
    decode_workspace_size,
    extend_partition_tokens,
    extend_workspace_size,
    paged_attn_decode,
    paged_attn_decode_noalloc,
    paged_attn_extend,
    paged_block_copy,
    paged_block_move,
    paged_kv_write,
)

__all__ = [
    "PkvError",
    "lib",
    "LIB_PATH",
    "cache_desc",
    "decode_partition_tokens",
    "decode_runs",
    "decode_workspace_size",
    "extend_partition_tokens",
    "extend_workspace_size",
    "paged_attn_decode",
    "paged_attn_decode_noalloc",
    "paged_attn_extend",
    "paged_block_copy",
    "paged_block_move",
    "paged_kv_write",
]
