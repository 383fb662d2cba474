"""The block masks the ring entry points build for all chunks in one launch, read back from
their workspace (ring_attn_fwd_masks / ring_attn_bwd_masks give the offsets) and compared bit for
bit with the oracle's tile classes, counts, lists and PARTIAL-tile bits of each chunk: the
ring-splash page's block mask (MaskInfo) of the Kvax page's create_attention_mask, one per KV
chunk, at the tile the kernels walk."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import ring_attention_merge_amd as ram
from ring_attention_merge_amd import workloads as wl

from gpu_util import mask_src, ring_desc, say

pytestmark = pytest.mark.gpu


def _chunk_allowed(w, c, b):
    """Element mask of batch row b against chunk c's keys (positions, segments and dense columns
    travel with the chunk)."""
    qp, kp = w.positions()
    ks = slice(c * w.chunk, (c + 1) * w.chunk)
    return oracle.allowed(qp[b], kp[b, ks], None if w.q_seg is None else w.q_seg[b],
                          None if w.kv_seg is None else w.kv_seg[b, ks], w.causal,
                          None if w.dense is None else w.dense[:, ks])


def _read(ws, off, count, dtype):
    nbytes = count * np.dtype(dtype).itemsize
    return ws[off:off + nbytes].cpu().numpy().view(dtype)


def _check_masks(w, ws, lay, what):
    n, B = w.n_chunks, w.B
    bq, bk, nQb, nKb = lay["block_q"], lay["block_kv"], lay["nQb"], lay["nKb"]
    T = B * nQb * nKb
    cls = _read(ws, lay["cls_off"], n * T, np.uint8).reshape(n, B, nQb, nKb)
    cnt = _read(ws, lay["cnt_off"], n * B * nQb, np.int32).reshape(n, B, nQb)
    col = _read(ws, lay["col_off"], n * T, np.int32).reshape(n, B, nQb, nKb)
    bits = None
    if lay["bits_off"] >= 0:
        W = bk // 32
        bits = _read(ws, lay["bits_off"], n * T * lay["tile_words"], np.uint32).reshape(n, B, nQb, nKb, bq, W)
    n_partial = 0
    for c in range(n):
        for b in range(B):
            ok = _chunk_allowed(w, c, b)
            rc, rn, ri = oracle.block_mask(ok, bq, bk)
            assert np.array_equal(cls[c, b], rc), f"{what}: classes of chunk {c} differ (b={b})"
            assert np.array_equal(cnt[c, b], rn), f"{what}: counts of chunk {c} differ (b={b})"
            assert np.array_equal(col[c, b], ri), f"{what}: lists of chunk {c} differ (b={b})"
            if bits is not None:
                part = rc == oracle.TILE_PARTIAL
                n_partial += int(part.sum())
                if part.any():
                    rb = oracle.partial_bits(ok, bq, bk)
                    assert np.array_equal(bits[c, b][part], rb[part]), f"{what}: bits of chunk {c} differ (b={b})"
    say(f"{what}: {n} chunks x {B} rows of {nQb}x{nKb} tiles at {bq}x{bk} bit-exact"
        + (f", {n_partial} PARTIAL tiles' bits" if bits is not None else ""))


def _dense_ring(seed=77):
    """A ring of 3 chunks of 384 keys, q shard 1 (positions 512..1023), with a dense mask over all
    1152 keys read per chunk at column c * 384."""
    w = wl.make("dense_ring", B=1, H=2, Hkv=1, Sq=512, chunk=384, n_chunks=3, D=128, q_shard=1, seed=seed)
    rng = np.random.default_rng(seed + 1)
    w.dense = wl.dense_mask(rng, 512, 1152, q_offset=512, window=96, n_global=40, block=64, p_block=0.2)
    return w


def _src(w, dev):
    src = mask_src(w, dev)
    if w.dense is not None:
        src.dense = torch.from_numpy(np.ascontiguousarray(w.dense)).to(dev)
        src.dense_chunk_step = w.chunk
    return src


FWD_CASES = {
    "c2_ring_shard": wl.c2_ring_shard,
    "c3_packed_docs": wl.c3_packed_docs,
    "c5_long_causal": wl.c5_long_causal,
    "dense_ring": _dense_ring,
}


@pytest.mark.parametrize("name", sorted(FWD_CASES))
def test_ring_fwd_masks_bitexact(name):
    w = FWD_CASES[name]()
    say(f"ring forward masks {name}: B={w.B} Sq={w.Sq} chunks {w.n_chunks} x {w.chunk}")
    dev = "cuda"
    d = ring_desc(w)
    src = _src(w, dev)
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    sinks = None if w.sinks is None else w.sinks.to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.Sq, dtype=torch.float32, device=dev)
    ws = torch.full((ram.ring_attn_workspace_bytes(d, w.n_chunks, src),), 0xCD, dtype=torch.uint8, device=dev)
    ram.ring_attn_fwd_1gpu(d, w.n_chunks, w.q_shard, q, k, v, src, sinks, out, lse, ws)
    torch.cuda.synchronize()
    lay = ram.ring_attn_fwd_masks(d, w.n_chunks, src)
    assert (lay["bits_off"] >= 0) == (w.dense is not None or w.q_seg is not None or w.kv_pos is not None)
    _check_masks(w, ws, lay, f"fwd {name}")
    if lay["order_off"] >= 0:
        # the rows the ring takes most tiles first: a permutation of the rows with non-increasing
        # total counts over the chunks
        rows = w.B * lay["nQb"]
        order = _read(ws, lay["order_off"], rows, np.int32)
        cnt = _read(ws, lay["cnt_off"], w.n_chunks * rows, np.int32).reshape(w.n_chunks, rows).sum(axis=0)
        assert np.array_equal(np.sort(order), np.arange(rows)), "row order is not a permutation"
        assert np.all(np.diff(np.minimum(cnt[order], 4095)) <= 0), "row order not by descending tile count"
        say(f"fwd {name}: row order of {rows} rows by descending tile count")


BWD_CASES = {
    "c2_ring_shard_s1024": lambda: wl.c2_ring_shard(Sq=1024, H=4, seed=91),
    "docs_s1024": lambda: wl.make("docs_s1024", B=2, H=2, Hkv=2, Sq=1024, chunk=256, n_chunks=4, D=128,
                                  docs=(64, 400, 0.05), seed=92),
    "dense_ring": _dense_ring,
}


@pytest.mark.parametrize("name", sorted(BWD_CASES))
def test_ring_bwd_masks_bitexact(name):
    w = BWD_CASES[name]()
    say(f"ring backward masks {name}: B={w.B} Sq={w.Sq} chunks {w.n_chunks} x {w.chunk}")
    dev = "cuda"
    d = ring_desc(w)
    src = _src(w, dev)
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.Sq, dtype=torch.float32, device=dev)
    fws = torch.empty(ram.ring_attn_workspace_bytes(d, w.n_chunks, src), dtype=torch.uint8, device=dev)
    ram.ring_attn_fwd_1gpu(d, w.n_chunks, w.q_shard, q, k, v, src, None, out, lse, fws)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(5)).to(q.dtype).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.full((ram.ring_attn_bwd_workspace_bytes(d, w.n_chunks, src),), 0xCD, dtype=torch.uint8, device=dev)
    ram.ring_attn_bwd_1gpu(d, w.n_chunks, w.q_shard, q, k, v, out, lse, dout, src, None, dq, dk, dv, None, ws)
    torch.cuda.synchronize()
    lay = ram.ring_attn_bwd_masks(d, w.n_chunks, src)
    assert (lay["bits_off"] >= 0) == (w.dense is not None)
    _check_masks(w, ws, lay, f"bwd {name}")
