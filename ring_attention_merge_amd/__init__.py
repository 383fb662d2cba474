"""Chunked (ring) attention forward for MI355X: HIP kernels behind a C ABI.

The work runs in libram.so (include/ram.h); this package is its ctypes
binding. Entry points carry the C names:
  build_block_mask, attn_fwd_chunk, lse_merge, ring_attn_fwd_1gpu,
  ring_attn_workspace_bytes, kernel_tile (ram_kernel_tile), and the backward:
  bwd_kernel_tile (ram_bwd_kernel_tile),
  attn_bwd_prep, attn_bwd_chunk, ring_attn_bwd_1gpu, ring_attn_bwd_workspace_bytes;
where the ring calls keep their block masks in the workspace: ring_attn_fwd_masks,
  ring_attn_bwd_masks; the ring without a workspace (static scratch): ring_attn_fwd_1gpu_noalloc;
and the measurement aids ram_mfma_probe (mfma_probe), the dense bf16 MFMA rate, and
ram_set_kernel_events (set_kernel_events), events around the ring's attention launches.
Build the library with ``python -m ring_attention_merge_amd.build``.
"""
from ._lib import (  # noqa: F401
    RAM_BF16, RAM_F32, RAM_OUT_MERGE, RAM_OUT_WRITE, RAM_PAD_SEGMENT_ID, RAM_TILE_EMPTY,
    RAM_TILE_FULL, RAM_TILE_PARTIAL, BlockMask, Desc, MaskSrc, RamError, alloc_block_mask,
    attn_bwd_chunk, attn_bwd_prep, attn_fwd_chunk, build_block_mask, bwd_kernel_tile, kernel_tile, load, lse_merge, mfma_probe,
    ring_attn_bwd_masks, ring_attn_fwd_masks,
    ring_attn_bwd_1gpu, ring_attn_bwd_workspace_bytes, ring_attn_fwd_1gpu, ring_attn_fwd_1gpu_noalloc,
    ring_attn_workspace_bytes,
    set_kernel_events)
