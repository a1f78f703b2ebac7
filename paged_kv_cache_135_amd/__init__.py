"""Paged KV cache hot path for AMD Instinct MI355X (gfx950).

* ``paged_kv_write`` / ``paged_attention_decode`` / ``paged_attention_decode_append`` /
  ``paged_attention_prefill`` / ``paged_kv_copy_blocks``: HIP kernels behind the C ABI of ``libpagedkv.so`` (declared in
  include/pagedkv.h), called with torch tensors.
* ``BlockPool``: host-side allocator producing block tables and slot mappings.
"""
from .binding import (DecodeLaunch, PagedKVError, PrefillLaunch, WriteLaunch, decode_order,
                      decode_workspace_bytes, load, noalloc_scratch_bytes, paged_attention_decode,
                      paged_attention_decode_append, paged_attention_decode_noalloc, paged_attention_decode_shared_prefix,
                      paged_attention_decode_shared_prefix_append, paged_attention_prefill, paged_kv_copy_blocks,
                      paged_kv_gather_blocks, paged_kv_scatter_blocks, paged_kv_write, read_probe,
                      tile_gather_probe,
                      swap_in_from_host, swap_out_to_host, tables_share_blocks,
                      validate_append_slots, validate_block_ids, validate_block_pairs,
                      validate_decode_inputs, validate_prefill_inputs, validate_seq_order,
                      validate_shared_prefix, validate_slots)
from .block_pool import BlockPool, OutOfBlocks, block_bytes, blocks_for_memory

__all__ = [
    "DecodeLaunch", "PrefillLaunch", "WriteLaunch", "PagedKVError", "BlockPool", "OutOfBlocks", "block_bytes",
    "blocks_for_memory", "decode_order", "decode_workspace_bytes", "load", "noalloc_scratch_bytes",
    "paged_attention_decode", "paged_attention_decode_append", "paged_attention_decode_noalloc", "paged_attention_decode_shared_prefix",
    "paged_attention_decode_shared_prefix_append", "paged_attention_prefill", "paged_kv_copy_blocks", "tables_share_blocks", "read_probe", "tile_gather_probe",
    "paged_kv_gather_blocks", "paged_kv_scatter_blocks", "paged_kv_write", "swap_in_from_host",
    "swap_out_to_host", "validate_append_slots", "validate_block_ids", "validate_block_pairs", "validate_decode_inputs",
    "validate_prefill_inputs", "validate_seq_order", "validate_shared_prefix", "validate_slots",
]
