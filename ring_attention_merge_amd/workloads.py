"""Seeded synthetic inputs for chunked (ring) attention.

This module holds no attention arithmetic. It only draws random numbers, rounds
the draws to the input dtype, and writes down the index bookkeeping that
describes a workload: document lengths, segment IDs, positions and chunk sizes.
The tests, the bench and the oracle checks all take their inputs from here, so
the HIP path and the oracle see the same values.

Layouts follow the Kvax page (flash_attention arguments): q is [B, Sq, H, D],
k and v are [B, Skv, Hkv, D], positions and segment IDs are [B, S] int32.
Padding tokens carry PAD_SEGMENT_ID. The Kvax page names the constant but does
not print its value; -1 is used, and generated document IDs are >= 0.

Recipe: ``np.random.default_rng(seed)``; draw order is document lengths (row by
row, packed-document workloads only), then q, k, v, then sinks. Values are
drawn in float32 and rounded to bfloat16 with round-to-nearest-even
(``torch.Tensor.to(torch.bfloat16)``) for bf16 workloads.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

PAD_SEGMENT_ID = -1


@dataclass
class Workload:
    """One attention workload: the q shard, the whole KV, and how KV is chunked.

    ``k``/``v`` hold all ``n_chunks * chunk`` keys. ``q_pos``/``kv_pos`` are
    None when positions are sequential (``q_pos_base + i`` and ``j`` over the
    concatenated KV); ``q_seg``/``kv_seg`` are None when there is no segment
    masking. ``q_shard`` is the ring index r of the q shard (its KV chunks are
    visited in ring order), or -1 for natural chunk order.
    """

    name: str
    B: int
    H: int
    Hkv: int
    Sq: int
    chunk: int
    n_chunks: int
    D: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    scale: float
    softcap: Optional[float]
    q_shard: int
    q_pos_base: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    sinks: Optional[torch.Tensor] = None
    q_pos: Optional[np.ndarray] = None
    kv_pos: Optional[np.ndarray] = None
    q_seg: Optional[np.ndarray] = None
    kv_seg: Optional[np.ndarray] = None
    dense: Optional[np.ndarray] = None   # uint8 [Sq, n_chunks*chunk], one mask over all keys
    meta: dict = field(default_factory=dict)

    @property
    def Skv(self) -> int:
        return self.chunk * self.n_chunks

    def positions(self):
        """Explicit position arrays ([B,Sq], [B,Skv] int64), sequential if unset."""
        qp = self.q_pos
        if qp is None:
            qp = np.broadcast_to(self.q_pos_base + np.arange(self.Sq), (self.B, self.Sq))
        kp = self.kv_pos
        if kp is None:
            kp = np.broadcast_to(np.arange(self.Skv), (self.B, self.Skv))
        return np.asarray(qp, np.int64), np.asarray(kp, np.int64)

    def as_f64(self):
        """q, k, v, sinks as float64 numpy arrays holding the rounded input values."""
        sinks = None if self.sinks is None else self.sinks.double().numpy()
        return (self.q.double().numpy(), self.k.double().numpy(), self.v.double().numpy(), sinks)


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def packed_documents(rng, B: int, S: int, len_lo: int, len_hi: int, pad_frac: float):
    """Segment IDs and positions for rows of packed documents plus trailing padding.

    Per row: document lengths are drawn from Uniform[len_lo, len_hi] (integers,
    inclusive) until the non-pad tokens are covered; the last document is cut to
    fit. Document IDs are 0, 1, 2, ...; positions restart at 0 in each document.
    The trailing round(pad_frac * S) tokens are padding: PAD_SEGMENT_ID with
    position 0.
    """
    n_pad = int(round(pad_frac * S))
    n_tok = S - n_pad
    seg = np.full((B, S), PAD_SEGMENT_ID, np.int32)
    pos = np.zeros((B, S), np.int32)
    lengths = []
    for b in range(B):
        t, doc, row = 0, 0, []
        while t < n_tok:
            L = int(rng.integers(len_lo, len_hi + 1))
            L = min(L, n_tok - t)
            seg[b, t:t + L] = doc
            pos[b, t:t + L] = np.arange(L, dtype=np.int32)
            row.append(L)
            t += L
            doc += 1
        lengths.append(row)
    return seg, pos, lengths


def dense_mask(rng, Sq: int, Skv: int, *, q_offset: int = 0, window: int = 256, n_global: int = 64,
               block: int = 128, p_block: float = 0.15, p_keep: float = 0.5, dead_rows: int = 3):
    """A seeded two-dimensional mask (uint8 [Sq, Skv], 1 = allowed) with the structures
    caller-given masks have: a band, global keys, random blocks and dead rows.

    Query i sits at key coordinate q_offset + i. The mask is the union of
      * a band: keys j with |q_offset + i - j| < window;
      * global keys: j < n_global;
      * random blocks: each (block x block) cell is picked with probability
        p_block; a picked cell is either all ones or, with probability 1/2,
        elements drawn independently with probability p_keep (cells are
        aligned to ``block`` from (0, 0), so with a tile that divides
        ``block`` they give whole FULL and ragged PARTIAL tiles);
    then ``dead_rows`` randomly chosen rows are cleared (rows with no key).
    Draw order: the cell picks, the all-ones / random choice per cell, the
    element draws of the random cells (row-major), then the dead rows.
    """
    m = np.zeros((Sq, Skv), dtype=bool)
    for i in range(Sq):                       # band, row by row (no [Sq, Skv] temporaries)
        c = q_offset + i
        lo, hi = max(0, c - window + 1), min(Skv, c + window)
        if lo < hi:
            m[i, lo:hi] = True
    m[:, :min(n_global, Skv)] = True
    nbq, nbk = -(-Sq // block), -(-Skv // block)
    pick = rng.random((nbq, nbk)) < p_block
    rand_cell = rng.random((nbq, nbk)) < 0.5
    for bi, bj in zip(*np.nonzero(pick)):
        r0, c0 = bi * block, bj * block
        r1, c1 = min(Sq, r0 + block), min(Skv, c0 + block)
        if rand_cell[bi, bj]:
            m[r0:r1, c0:c1] |= rng.random((r1 - r0, c1 - c0)) < p_keep
        else:
            m[r0:r1, c0:c1] = True
    if dead_rows and Sq:
        m[rng.choice(Sq, size=min(dead_rows, Sq), replace=False)] = False
    return m.view(np.uint8)


def make(name: str, *, B: int, H: int, Hkv: int, Sq: int, chunk: int, n_chunks: int, D: int,
         dtype: str = "bf16", causal: bool = True, softcap: Optional[float] = None,
         with_sinks: bool = False, q_shard: int = -1, seed: int = 0,
         docs: Optional[tuple] = None, v_uniform: bool = False,
         scale: Optional[float] = None) -> Workload:
    """Build a workload from the recipe in the module docstring.

    ``docs=(len_lo, len_hi, pad_frac)`` makes packed documents (self-attention:
    q and KV share the segment IDs and positions, so ``Sq`` must equal the KV
    length). ``q_shard=r`` places the q shard at ring index r, so sequential q
    positions start at ``r * Sq``.
    """
    rng = np.random.default_rng(seed)
    Skv = chunk * n_chunks
    q_seg = kv_seg = q_pos = kv_pos = None
    meta = {}
    if docs is not None:
        if Sq != Skv:
            raise ValueError("packed documents need Sq == total KV length")
        seg, pos, lengths = packed_documents(rng, B, Sq, docs[0], docs[1], docs[2])
        q_seg = kv_seg = seg
        q_pos = kv_pos = pos
        meta["doc_lengths"] = lengths
    q = rng.standard_normal((B, Sq, H, D), dtype=np.float32)
    k = rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32)
    if v_uniform:
        v = rng.uniform(-1.0, 1.0, size=(B, Skv, Hkv, D)).astype(np.float32)
    else:
        v = rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32)
    sinks = None
    if with_sinks:
        sinks = torch.from_numpy(rng.standard_normal(H, dtype=np.float32))
    q_pos_base = q_shard * Sq if q_shard >= 0 else 0
    return Workload(
        name=name, B=B, H=H, Hkv=Hkv, Sq=Sq, chunk=chunk, n_chunks=n_chunks, D=D, dtype=dtype,
        causal=causal, scale=(1.0 / math.sqrt(D)) if scale is None else scale, softcap=softcap,
        q_shard=q_shard, q_pos_base=q_pos_base, q=_round(q, dtype), k=_round(k, dtype),
        v=_round(v, dtype), sinks=sinks, q_pos=q_pos, kv_pos=kv_pos, q_seg=q_seg, kv_seg=kv_seg,
        meta=meta)


# The five workloads, with the sizes they are specified at.
def c1_causal_f32() -> Workload:
    """Causal self-attention, B=1 H=2 S=256 D=64, fp32, one KV chunk."""
    return make("c1_causal_f32_s256", B=1, H=2, Hkv=2, Sq=256, chunk=256, n_chunks=1, D=64,
                dtype="f32", seed=1001)


def c2_ring_shard(Sq: int = 4096, H: int = 8, n_chunks: int = 4, seed: int = 1002) -> Workload:
    """Ring shard 3 of 4: local q of Sq rows at positions 3*Sq.., KV of 4 chunks of Sq."""
    return make(f"c2_ring_shard3of4_s{Sq}", B=1, H=H, Hkv=H, Sq=Sq, chunk=Sq, n_chunks=n_chunks,
                D=128, q_shard=n_chunks - 1, seed=seed)


def c3_packed_docs(S: int = 8192, B: int = 2, H: int = 16, len_lo: int = 128, len_hi: int = 2048,
                   seed: int = 1003) -> Workload:
    """Packed documents with 5% trailing padding, one KV chunk, causal within documents."""
    return make(f"c3_packed_docs_s{S}", B=B, H=H, Hkv=H, Sq=S, chunk=S, n_chunks=1, D=128,
                docs=(len_lo, len_hi, 0.05), seed=seed)


def c4_gqa_cap_sinks(S: int = 16384, H: int = 32, Hkv: int = 8, n_chunks: int = 4,
                     seed: int = 1004) -> Workload:
    """GQA (or MQA with Hkv=1), soft cap 50, per-head sinks on the first chunk."""
    return make(f"c4_gqa_h{H}_hkv{Hkv}_s{S}", B=1, H=H, Hkv=Hkv, Sq=S, chunk=S // n_chunks,
                n_chunks=n_chunks, D=128, softcap=50.0, with_sinks=True, seed=seed)


def c5_long_causal(S: int = 32768, H: int = 32, Hkv: int = 8, n_chunks: int = 8,
                   seed: int = 1005) -> Workload:
    """Long-context causal, 8 sequential chunks merged by LSE, v ~ U(-1, 1)."""
    return make(f"c5_long_causal_h{H}_hkv{Hkv}_s{S}", B=1, H=H, Hkv=Hkv, Sq=S,
                chunk=S // n_chunks, n_chunks=n_chunks, D=128, v_uniform=True, seed=seed)


def c5_dense(S: int = 32768, H: int = 32, Hkv: int = 8, n_chunks: int = 8, seed: int = 1006) -> Workload:
    """The long-context causal workload with a dense two-dimensional mask over all keys:
    a band of 2048 around the diagonal, 256 global keys, 10% of the 512x512 cells picked
    (half of them all ones, half with elements kept at p = 1/2) and 3 cleared rows, ANDed
    with the causal test. The mask is drawn after q, k, v from the same generator."""
    w = make(f"c5_dense_h{H}_hkv{Hkv}_s{S}", B=1, H=H, Hkv=Hkv, Sq=S, chunk=S // n_chunks,
             n_chunks=n_chunks, D=128, v_uniform=True, seed=seed)
    rng = np.random.default_rng(seed + 1_000_000)
    w.dense = dense_mask(rng, S, S, window=2048, n_global=256, block=512, p_block=0.1, p_keep=0.5,
                         dead_rows=3)
    return w


def sampled_rows(Sq: int, chunk: int, n: int = 256, seed: int = 1005) -> np.ndarray:
    """Query rows checked at full size: fixed edge rows plus seeded random ones.

    Always includes rows 0, 1, 127, 128, every chunk edge (chunk*c - 1 and
    chunk*c) and the last row; the rest are drawn from ``default_rng(seed)``.
    """
    fixed = {0, 1, 127, 128, Sq - 1}
    for c in range(1, Sq // chunk + 1):
        fixed.add(min(Sq - 1, chunk * c - 1))
        if chunk * c < Sq:
            fixed.add(chunk * c)
    fixed = sorted(r for r in fixed if 0 <= r < Sq)
    rng = np.random.default_rng(seed)
    rest = [r for r in rng.permutation(Sq) if r not in set(fixed)]
    rows = fixed + rest[: max(0, n - len(fixed))]
    return np.array(sorted(rows), dtype=np.int64)
