"""Seeded synthetic decode workloads for the paged KV-cache path.

This package builds inputs only: sequence lengths, pools, block tables,
queries, cache contents, new-token rows, slot mappings and copy-on-write
pairs, for decode batches and for prefill / chunked-extend batches.  It
holds none of the attention arithmetic and imports neither the oracle nor
the HIP binding, so both sides can be fed from it.
"""

from .configs import CONFIGS, DecodeConfig, get_config, scaled
from .generate import (
    Layout,
    Workload,
    build_layout,
    decode_slots,
    cow_layout,
    generate_host,
    generate_device,
    f32_to_bf16_bits,
)
from .extend import (
    EXTEND_CONFIGS,
    ExtendConfig,
    ExtendWorkload,
    extend_layout,
    extend_slots,
    generate_extend_device,
    generate_extend_host,
    get_extend_config,
)

__all__ = [
    "CONFIGS",
    "DecodeConfig",
    "get_config",
    "scaled",
    "Layout",
    "Workload",
    "build_layout",
    "decode_slots",
    "cow_layout",
    "generate_host",
    "generate_device",
    "f32_to_bf16_bits",
    "EXTEND_CONFIGS",
    "ExtendConfig",
    "ExtendWorkload",
    "extend_layout",
    "extend_slots",
    "generate_extend_device",
    "generate_extend_host",
    "get_extend_config",
]
