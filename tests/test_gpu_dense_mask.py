"""GPU parity of the dense two-dimensional mask path against the float64 oracle.

The builder's classes, tile lists and PARTIAL-tile bits are compared bit for
bit with oracle.block_mask / oracle.partial_bits of the oracle's element mask;
attention outputs at the tolerances of gpu_util (out 2e-2 bf16 / 1e-4 fp32,
lse 1e-3, empty rows exactly (0, -inf)). Outputs are poisoned with NaN first.
Masks come from workloads.dense_mask (band, global keys, random blocks with
random elements, dead rows).
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import ring_attention_merge_amd as ram
from ring_attention_merge_amd import workloads as wl
from gpu_util import compare, ring_by_chunks, ring_splits, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
POISON = 0x5A5A5A5A


def _i32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


# ------------------------------------------------------------------------------ block mask + bits
BM_CASES = {
    # name: B, Sq, Skv, causal, q_base, extra ("docs" / "shuffle" / None), dense_ld pad (None: no dense mask)
    "dense_noncausal": (1, 300, 260, False, 0, None, 0),
    "dense_causal_offset": (2, 257, 390, True, 133, None, 17),
    "dense_docs": (2, 400, 400, True, 0, "docs", 0),
    "dense_shuffled_pos": (1, 190, 230, True, 0, "shuffle", 5),
    "dense_long_rows": (1, 150, 2500, True, 2000, None, 3),
    "bits_only_causal": (1, 300, 280, True, 100, None, None),
    "bits_only_docs": (2, 333, 333, True, 0, "docs", None),
}
BM_TILES = [(128, 64), (64, 32), (16, 16), (48, 80), (256, 512)]


@pytest.mark.parametrize("tile", BM_TILES, ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("name", sorted(BM_CASES))
def test_block_mask_dense_bits_bitexact(name, tile):
    B, Sq, Skv, causal, qb, extra, pad = BM_CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    say(f"block mask dense {name} tile {tile}")
    dense = wl.dense_mask(rng, Sq, Skv, q_offset=qb, window=40, n_global=9, block=48)
    ld = Skv + (pad or 0)
    dense_ld = np.zeros((Sq, ld), np.uint8)
    dense_ld[:, :Skv] = dense * rng.integers(1, 255, size=dense.shape)   # any nonzero byte allows
    dense_ld[:, Skv:] = 1                                                  # never read
    if pad is None:
        dense = None
    qp = kp = qs = ks = None
    if extra == "docs":
        qs, qp, _ = wl.packed_documents(rng, B, Sq, 20, 150, 0.05)
        ks, kp = qs, qp
    elif extra == "shuffle":
        qp = rng.integers(0, 300, size=(B, Sq)).astype(np.int32)
        kp = rng.integers(0, 300, size=(B, Skv)).astype(np.int32)
    d = ram.Desc(B=B, Sq=Sq, Skv=Skv, H=1, Hkv=1, D=128, causal=causal, block_q=tile[0], block_kv=tile[1])
    src = ram.MaskSrc(q_pos=_i32(qp), kv_pos=_i32(kp), q_seg=_i32(qs), kv_seg=_i32(ks), q_pos_base=qb,
                      dense=None if dense is None else _u8(dense_ld), dense_ld=ld if pad else 0)
    bm = ram.alloc_block_mask(d, with_bits=True)
    bm.tile_class.fill_(0xAB)
    bm.row_cnt.fill_(-7)
    bm.col_idx.fill_(-7)
    bm.bits.fill_(POISON)
    ram.build_block_mask(d, src, bm)
    torch.cuda.synchronize()
    nQb, nKb, W = bm.nQb, bm.nKb, -(-tile[1] // 32)
    cls = bm.tile_class.cpu().numpy()[: B * nQb * nKb].reshape(B, nQb, nKb)
    cnt = bm.row_cnt.cpu().numpy()[: B * nQb].reshape(B, nQb)
    col = bm.col_idx.cpu().numpy()[: B * nQb * nKb].reshape(B, nQb, nKb)
    bits = bm.bits.cpu().numpy().view(np.uint32)[: B * nQb * nKb * tile[0] * W].reshape(B, nQb, nKb, tile[0], W)
    n_partial = 0
    for b in range(B):
        qpb = qp[b] if qp is not None else qb + np.arange(Sq)
        kpb = kp[b] if kp is not None else np.arange(Skv)
        ok = oracle.allowed(qpb, kpb, None if qs is None else qs[b], None if ks is None else ks[b], causal,
                            dense=dense)
        rc, rn, ri = oracle.block_mask(ok, tile[0], tile[1])
        rb = oracle.partial_bits(ok, tile[0], tile[1])
        assert np.array_equal(cls[b], rc), f"classes differ (b={b})"
        assert np.array_equal(cnt[b], rn), f"row counts differ (b={b})"
        assert np.array_equal(col[b], ri), f"tile lists differ (b={b})"
        part = rc == oracle.TILE_PARTIAL
        n_partial += int(part.sum())
        assert np.array_equal(bits[b][part], rb[part]), f"PARTIAL tile bits differ (b={b})"
        assert np.all(bits[b][~part] == POISON), f"bits written outside PARTIAL tiles (b={b})"
    assert n_partial > 0


# ------------------------------------------------------------------------------ one chunk
CHUNK_CASES = {
    # name: dtype, D, B, Sq, Skv, H, Hkv, causal, q_base, segments, cap, sinks
    "bf16_d128_noncausal": ("bf16", 128, 1, 384, 320, 4, 2, False, 0, False, None, False),
    "bf16_d128_causal_ragged_sinks": ("bf16", 128, 2, 300, 333, 2, 1, True, 100, False, None, True),
    "bf16_d64_segs_cap": ("bf16", 64, 1, 260, 260, 4, 4, True, 0, True, 5.0, True),
    "bf16_d128_cap_mqa": ("bf16", 128, 1, 256, 448, 8, 1, False, 0, False, 30.0, False),
    "f32_d128_causal_segs": ("f32", 128, 1, 200, 257, 2, 2, True, 57, True, None, True),
    "f32_d64_noncausal_cap": ("f32", 64, 2, 131, 190, 6, 3, False, 0, False, 3.0, False),
}


@pytest.mark.parametrize("name", sorted(CHUNK_CASES))
def test_chunk_dense(name):
    dt, D, B, Sq, Skv, H, Hkv, causal, qb, segs, cap, with_sinks = CHUNK_CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    q = torch.from_numpy(rng.standard_normal((B, Sq, H, D), dtype=np.float32)).to(tdt)
    k = torch.from_numpy(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32)).to(tdt)
    v = torch.from_numpy(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32)).to(tdt)
    sinks = torch.from_numpy(rng.standard_normal(H, dtype=np.float32)) if with_sinks else None
    dense = wl.dense_mask(rng, Sq, Skv, q_offset=qb, window=70, n_global=5, block=64)
    qs = ks = None
    if segs:
        qs = rng.integers(-1, 3, size=(B, Sq)).astype(np.int32)
        ks = rng.integers(-1, 3, size=(B, Skv)).astype(np.int32)
        qs[:, : Sq // 2] = 1
        ks[:, : Skv // 2] = 1
    say(f"attn_fwd_chunk dense {name}")
    dcode = ram.RAM_BF16 if dt == "bf16" else ram.RAM_F32
    bq, bk = ram.kernel_tile(dcode, D)
    d = ram.Desc(B=B, Sq=Sq, Skv=Skv, H=H, Hkv=Hkv, D=D, dtype=dcode, scale=1.0 / math.sqrt(D), softcap=cap or 0.0,
                 causal=causal, block_q=bq, block_kv=bk)
    src = ram.MaskSrc(q_pos_base=qb, q_seg=_i32(qs), kv_seg=_i32(ks), dense=_u8(dense))
    bm = ram.alloc_block_mask(d, with_bits=True)
    out = torch.full((B, Sq, H, D), float("nan"), device=DEV)
    lse = torch.full((B, H, Sq), float("nan"), device=DEV)
    ram.build_block_mask(d, src, bm)
    ram.attn_fwd_chunk(d, q.to(DEV), k.to(DEV), v.to(DEV), src, bm, None if sinks is None else sinks.to(DEV), 0,
                       out, lse)
    torch.cuda.synchronize()
    qp = np.broadcast_to(qb + np.arange(Sq), (B, Sq))
    kp = np.broadcast_to(np.arange(Skv), (B, Skv))
    ro, rl = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale=d.scale,
                              q_pos=qp, kv_pos=kp, q_seg=qs, kv_seg=ks, causal=causal, softcap=cap,
                              sinks=None if sinks is None else sinks.double().numpy(), dense=dense)
    assert (~dense.any(axis=1)).any(), "no cleared row exercised"
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, dt, "dense chunk " + name)


# ------------------------------------------------------------------------------ ring
RING_CASES = {
    # name: dtype, D, B, H, Hkv, Sq, chunk, n, q_shard, causal, step ("global" / "reuse"), ld pad, cap, sinks
    "global_shard3of4": ("bf16", 128, 1, 4, 2, 256, 256, 4, 3, True, "global", 0, None, True),
    "global_noncausal_ragged": ("bf16", 128, 2, 2, 1, 200, 150, 3, 1, False, "global", 7, 20.0, False),
    "reuse_noncausal_shard2of4": ("bf16", 128, 1, 4, 4, 256, 256, 4, 2, False, "reuse", 0, None, True),
    "reuse_noncausal_d64_pad": ("bf16", 64, 1, 2, 2, 190, 190, 3, 0, False, "reuse", 33, 4.0, False),
    "global_f32_d64": ("f32", 64, 1, 2, 2, 130, 128, 2, -1, True, "global", 0, None, True),
}


@pytest.mark.parametrize("name", sorted(RING_CASES))
def test_ring_dense(name):
    dt, D, B, H, Hkv, Sq, C, n, r, causal, kind, pad, cap, with_sinks = RING_CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    w = wl.make(name, B=B, H=H, Hkv=Hkv, Sq=Sq, chunk=C, n_chunks=n, D=D, dtype=dt, causal=causal,
                softcap=cap, with_sinks=with_sinks, q_shard=r, seed=zlib.crc32(name.encode()) % 1000)
    step = C if kind == "global" else 0
    cols = C + (n - 1) * step
    dense = wl.dense_mask(rng, Sq, cols, q_offset=w.q_pos_base if kind == "global" else 0, window=60,
                          n_global=3, block=64)
    ld = cols + pad
    dpad = np.ones((Sq, ld), np.uint8)
    dpad[:, :cols] = dense
    say(f"ring dense {name}: {kind} step={step} ld={ld} order shard={r}")
    d = ram.Desc(B=B, Sq=Sq, Skv=C, H=H, Hkv=Hkv, D=D, dtype=ram.RAM_BF16 if dt == "bf16" else ram.RAM_F32,
                 scale=w.scale, softcap=cap or 0.0, causal=causal)
    src = ram.MaskSrc(dense=_u8(dpad), dense_ld=ld if pad else 0, dense_chunk_step=step)
    out = torch.full((B, Sq, H, D), float("nan"), device=DEV).to(w.q.dtype)
    lse = torch.full((B, H, Sq), float("nan"), device=DEV)
    ws = torch.empty(ram.ring_attn_workspace_bytes(d, n, src), dtype=torch.uint8, device=DEV)
    sinks = None if w.sinks is None else w.sinks.to(DEV)
    ram.ring_attn_fwd_1gpu(d, n, r, w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), src, sinks, out, lse, ws)
    # the same ring as attn_fwd_chunk calls in ring order: bit-identical with one workgroup per row
    # of q tiles (and for the one-chunk-per-launch kernels), equal up to the merge order's
    # rounding when the ring splits each row's visits over two workgroups
    o2, l2 = ring_by_chunks(d, n, r, w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), src, sinks)
    torch.cuda.synchronize()
    o2 = o2.to(out.dtype)
    if ring_splits(d, n):
        torch.testing.assert_close(out.float(), o2.float(), rtol=0, atol=2e-2)
        fin = torch.isfinite(l2)
        assert torch.equal(fin, torch.isfinite(lse))
        torch.testing.assert_close(lse[fin], l2[fin], rtol=0, atol=1e-4)
    else:
        assert torch.equal(out, o2) and torch.equal(lse, l2), "one-launch ring differs from chunk calls"
    q, k, v, s64 = w.as_f64()
    qp, kp = w.positions()
    order = [(r - t) % n for t in range(n)] if r >= 0 else list(range(n))
    ro, rl = oracle.chunked(q, k, v, scale=w.scale, q_pos=qp, kv_pos=kp,
                            bounds=[(c * C, (c + 1) * C) for c in range(n)], order=order, causal=causal,
                            softcap=cap, sinks=s64, dense=dense, dense_col0=[c * step for c in range(n)])
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, dt, "dense ring " + name)


def test_ring_dense_c2_shape_sampled():
    """The 4-step ring shard (local Sq 4096 as shard 3 of 4, 4 chunks of 4096, H=8, D=128, bf16)
    with one dense mask over all 16384 keys, checked on sampled rows."""
    w = wl.c2_ring_shard()
    rng = np.random.default_rng(2002)
    dense = wl.dense_mask(rng, w.Sq, w.Skv, q_offset=w.q_pos_base, window=512, n_global=128, block=256,
                          p_block=0.1, dead_rows=4)
    say(f"ring dense {w.name}: dense [{w.Sq}, {w.Skv}]")
    d = ram.Desc(B=1, Sq=w.Sq, Skv=w.chunk, H=w.H, Hkv=w.Hkv, D=128, scale=w.scale, causal=True)
    src = ram.MaskSrc(dense=_u8(dense), dense_chunk_step=w.chunk)
    out = torch.full((1, w.Sq, w.H, 128), float("nan"), device=DEV).to(torch.bfloat16)
    lse = torch.full((1, w.H, w.Sq), float("nan"), device=DEV)
    ws = torch.empty(ram.ring_attn_workspace_bytes(d, w.n_chunks, src), dtype=torch.uint8, device=DEV)
    ram.ring_attn_fwd_1gpu(d, w.n_chunks, w.q_shard, w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), src, None, out, lse, ws)
    torch.cuda.synchronize()
    dead = np.nonzero(~dense.any(axis=1))[0]
    rows = np.unique(np.concatenate([wl.sampled_rows(w.Sq, 1024, n=256, seed=2002), dead]))
    q, k, v, _ = w.as_f64()
    qp, kp = w.positions()
    ro, rl = oracle.attention(q, k, v, scale=w.scale, q_pos=qp, kv_pos=kp, causal=True, dense=dense, rows=rows)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", "c2 shape dense", rows=rows)


def test_c5dense_full_sampled():
    """The long-context causal workload with its dense mask over all 32768 keys (the bench's
    c5dense: 8 chunks of 4096, H=32 over Hkv=8, D=128, bf16), at full size, checked on sampled
    rows plus the mask's dead rows."""
    w = wl.c5_dense()
    say(f"ring dense {w.name}: dense [{w.Sq}, {w.Skv}], {w.n_chunks} chunks")
    d = ram.Desc(B=1, Sq=w.Sq, Skv=w.chunk, H=w.H, Hkv=w.Hkv, D=128, scale=w.scale, causal=True)
    src = ram.MaskSrc(dense=_u8(w.dense), dense_chunk_step=w.chunk)
    out = torch.full((1, w.Sq, w.H, 128), float("nan"), device=DEV).to(torch.bfloat16)
    lse = torch.full((1, w.H, w.Sq), float("nan"), device=DEV)
    ws = torch.empty(ram.ring_attn_workspace_bytes(d, w.n_chunks, src), dtype=torch.uint8, device=DEV)
    ram.ring_attn_fwd_1gpu(d, w.n_chunks, w.q_shard, w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), src, None, out, lse, ws)
    torch.cuda.synchronize()
    dead = np.nonzero(~w.dense.any(axis=1))[0]
    rows = np.unique(np.concatenate([wl.sampled_rows(w.Sq, w.chunk, n=128, seed=2006), dead]))
    q, k, v, _ = w.as_f64()
    qp, kp = w.positions()
    ro, rl = oracle.attention(q, k, v, scale=w.scale, q_pos=qp, kv_pos=kp, causal=True, dense=w.dense, rows=rows)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", "c5dense full", rows=rows)
