"""Paged KV-cache write path for AMD Instinct MI355X (gfx950).

The compute lives in libkvw.so (HIP, built from csrc/kvw.hip; C-ABI in
include/kvw.h).  This package only builds and binds it.
"""
from .kvw import (  # noqa: F401
    KVW_FLAG_BAD_BLOCK,
    KVW_FLAG_COUNT,
    KVW_FLAG_NUM_TOKENS,
    KVW_FLAG_SLOT_OOB,
    KVW_PAD_ID,
    KVW_SCHEDULE_AUTO,
    KVW_SCHEDULE_ONE_KERNEL,
    KVW_SCHEDULE_TWO_KERNELS,
    KVW_SLOTS_PAGED,
    KVW_SLOTS_PRECOMPUTED,
    KVW_SLOTS_RANGES,
    KvwError,
    kvw_decode_attention,
    kvw_decode_attention_noalloc,
    kvw_decode_merge,
    kvw_decode_workspace_size,
    kvw_kv_write,
    kvw_map_ranges_to_kernel_blocks,
    kvw_map_to_kernel_blocks,
    kvw_ranges_to_block_table,
    kvw_slot_mapping_paged,
    kvw_slot_mapping_ranges,
    library,
)
