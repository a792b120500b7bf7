"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

A thin Python binding over ``libpkv.so`` (C ABI in ``include/pkv.h`` and
``include/pkv_block_manager.h``): argument marshalling only, every step of the
path runs in the library's HIP kernels or its native block manager.  The
library must be built first (``python -m paged_kv_cache_200_amd.build``);
using the ops without it raises.
"""

from .ops import (  # noqa: F401
    BLOCK_SIZE,
    DecodeStep,
    IN_PASS_MERGE_MAX_PARTITIONS,
    append_paged_decode,
    append_paged_decode_layers,
    append_paged_decode_planned,
    append_paged_decode_static,
    STATIC_SCRATCH_BYTES,
    append_paged_decode_shared_prefix,
    copy_blocks,
    decode_engine,
    decode_partition_size,
    decode_plan,
    decode_workspace_bytes,
    describe_device_error,
    device_error,
    kv_append,
    lse_combine,
    paged_decode,
    paged_decode_partials,
    paged_decode_planned,
    paged_decode_shared_prefix,
    paged_prefill,
    shared_prefix_workspace_bytes,
)
from .block_manager import BlockManager, OutOfBlocks  # noqa: F401

__version__ = "1.0.0"
