"""Float64 CPU oracle for chunked (ring) attention. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package. The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

Contents:
  attention.attention    plain masked softmax attention, full score matrix
  attention.allowed      the element mask from positions, segment IDs and a dense mask
  attention.merge        the sigmoid/softplus LSE merge
  attention.chunked      attention per KV chunk folded with ``merge``
  attention.attention_bwd  gradients of ``attention`` (q, k, v, sinks)
  attention.chunked_bwd  the ring backward: chunk gradients against the final out / lse
  blockmask.block_mask   tile classes and compacted non-empty tile lists
  blockmask.partial_bits the element mask of each PARTIAL tile as bits

Every function is pinned by tests under ``tests/test_oracle_*.py`` against
closed forms, library routines, brute force and invariants; the soft-cap
formula itself is a reading (the pages give only the parameter), pinned to its
closed form and its large-cap limit, but not to any value on the pages.
"""
from .attention import (allowed, attention, attention_bwd, attention_dq, merge, chunked, chunked_bwd,
                        DEFAULT_MASK_VALUE, PAD_SEGMENT_ID)
from .blockmask import block_mask, partial_bits, TILE_EMPTY, TILE_PARTIAL, TILE_FULL

__all__ = ["allowed", "attention", "attention_bwd", "attention_dq", "merge", "chunked", "chunked_bwd", "block_mask", "partial_bits", "DEFAULT_MASK_VALUE",
           "PAD_SEGMENT_ID", "TILE_EMPTY", "TILE_PARTIAL", "TILE_FULL"]
