"""Tile classification and compacted non-empty tile lists. TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline may use this.

Sources: the ejkernel ring-splash source page names block-sparse mask metadata
(a per-tile block mask plus lists of the tiles to visit) without defining it;
the Kvax page's create_attention_mask builds block-wise masks from positions
and segment IDs and skips blocks with nothing to attend. Reading: a tile is
EMPTY when none of its (query, key) pairs is allowed, FULL when all are, else
PARTIAL; tiles are clipped at the sequence ends (pairs past the end do not
count). Each row of tiles lists its non-EMPTY key tiles in ascending order;
list slots past the count hold -1.

The ring-splash page's make_ring_attention also keeps, for the tiles a mask
only partly allows, the contents of that partial block (MaskInfo's
partial_mask_blocks, reached through mask_next). Reading: the contents are the
tile's element mask as bits, one row of ceil(block_kv / 32) 32-bit words per
query row of the tile, key j of the tile at bit j % 32 of word j // 32; rows
and keys past the sequence ends read 0. They are kept for PARTIAL tiles only;
every other tile reads all zeros here.
"""
from __future__ import annotations

import numpy as np

TILE_EMPTY, TILE_PARTIAL, TILE_FULL = 0, 1, 2


def block_mask(ok, block_q, block_kv):
    """Classify the tiles of one element mask ``ok`` [Sq, Skv] (bool).

    Returns (tile_class uint8 [nQb, nKb], row_cnt int32 [nQb],
    col_idx int32 [nQb, nKb]) with nQb = ceil(Sq/block_q), nKb = ceil(Skv/block_kv).
    """
    ok = np.asarray(ok, dtype=bool)
    Sq, Skv = ok.shape
    nQb = -(-Sq // block_q)
    nKb = -(-Skv // block_kv)
    cls = np.zeros((nQb, nKb), np.uint8)
    for qb in range(nQb):
        rows = ok[qb * block_q:(qb + 1) * block_q]
        for kb in range(nKb):
            tile = rows[:, kb * block_kv:(kb + 1) * block_kv]
            if tile.all():
                cls[qb, kb] = TILE_FULL
            elif tile.any():
                cls[qb, kb] = TILE_PARTIAL
    row_cnt = np.zeros(nQb, np.int32)
    col_idx = np.full((nQb, nKb), -1, np.int32)
    for qb in range(nQb):
        nz = [kb for kb in range(nKb) if cls[qb, kb] != TILE_EMPTY]
        row_cnt[qb] = len(nz)
        col_idx[qb, :len(nz)] = nz
    return cls, row_cnt, col_idx


def partial_bits(ok, block_q, block_kv):
    """Bit contents of the PARTIAL tiles of one element mask ``ok`` [Sq, Skv].

    Returns uint32 [nQb, nKb, block_q, ceil(block_kv/32)]: for a PARTIAL tile,
    bit j % 32 of word j // 32 in row i is ok[qb*block_q + i, kb*block_kv + j]
    (0 past the ends); all words of EMPTY and FULL tiles are 0.
    """
    ok = np.asarray(ok, dtype=bool)
    Sq, Skv = ok.shape
    cls, _, _ = block_mask(ok, block_q, block_kv)
    nQb, nKb = cls.shape
    W = -(-block_kv // 32)
    bits = np.zeros((nQb, nKb, block_q, W), np.uint32)
    for qb in range(nQb):
        for kb in range(nKb):
            if cls[qb, kb] != TILE_PARTIAL:
                continue
            for i in range(min(block_q, Sq - qb * block_q)):
                for j in range(min(block_kv, Skv - kb * block_kv)):
                    if ok[qb * block_q + i, kb * block_kv + j]:
                        bits[qb, kb, i, j // 32] |= np.uint32(1 << (j % 32))
    return bits
