"""Randomized parity sweep of ring_attn_fwd_1gpu against the float64 oracle.

Seeded random small rings crossing the features the fixed cases test one by one: batch rows,
kv-head grouping (GQA / MQA), head dim, dtype, ragged query and chunk lengths, chunk count and
ring shard, causal or not, soft cap, sinks, packed documents (segment IDs and positions that
restart per document), and dense masks read either over all keys or reused at every step. A
few cases have Sq * H / Hkv >= 32768, where the ring reads V repacked. Each case is compared
element by element with oracle.chunked (the pages' per-chunk attention folded by the LSE
merge) at the stated tolerances; the seed names the case."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import ring_attention_merge_amd as ram
from ring_attention_merge_amd import workloads as wl
from gpu_util import compare, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 100
N_PACKED_V = 5


def _case(seed: int, large: bool = False) -> dict:
    rng = np.random.default_rng(70_000 + seed)
    if large:
        # large enough for the repacked-V path: Sq * H / Hkv >= 32768, no soft cap
        n = int(rng.integers(1, 4))
        return dict(dtype="bf16", D=128, B=1, Hkv=1, H=8, Sq=4096, chunk=int(rng.integers(200, 700)), n=n,
                    q_shard=int(rng.integers(-1, n)), causal=bool(rng.random() < 0.7), cap=None,
                    sinks=bool(rng.random() < 0.5), feature="dense" if rng.random() < 0.4 else "plain",
                    reuse=bool(rng.random() < 0.3), seed=seed)
    feature = str(rng.choice(["plain", "docs", "dense"], p=[0.5, 0.25, 0.25]))
    dtype = "f32" if rng.random() < 0.15 else "bf16"
    n = int(rng.integers(1, 5))
    c = dict(dtype=dtype, D=64 if rng.random() < 0.3 else 128, B=int(rng.integers(1, 3)),
             Hkv=int(rng.choice([1, 2, 4])), n=n, causal=bool(rng.random() < 0.7),
             cap=float(rng.uniform(2.0, 60.0)) if rng.random() < 0.3 else None, sinks=bool(rng.random() < 0.3),
             feature=feature, reuse=bool(rng.random() < 0.3), seed=seed)
    c["H"] = c["Hkv"] * int(rng.choice([1, 2, 4]))
    if feature == "docs":
        c["chunk"] = int(rng.integers(16, 400))
        c["Sq"] = c["chunk"] * n
        c["q_shard"] = -1
    else:
        c["chunk"] = int(rng.integers(1, 500))
        c["Sq"] = int(rng.integers(1, 600))
        c["q_shard"] = int(rng.integers(-1, n))
    return c


@pytest.mark.parametrize("seed", list(range(N_CASES + N_PACKED_V)))
def test_random_ring(seed):
    check_ring(seed, _case(seed, large=seed >= N_CASES))


def check_ring(seed: int, c: dict):
    """One random ring forward against the oracle (the case drawn by _case)."""
    docs = (16, max(32, c["Sq"] // 2), 0.05) if c["feature"] == "docs" else None
    w = wl.make(f"rand{seed}", B=c["B"], H=c["H"], Hkv=c["Hkv"], Sq=c["Sq"], chunk=c["chunk"], n_chunks=c["n"],
                D=c["D"], dtype=c["dtype"], causal=c["causal"], softcap=c["cap"], with_sinks=c["sinks"],
                q_shard=c["q_shard"], docs=docs, seed=seed)
    C, n, r = c["chunk"], c["n"], c["q_shard"]
    dense, step = None, 0
    if c["feature"] == "dense":
        rng = np.random.default_rng(90_000 + seed)
        step = 0 if c["reuse"] else C
        cols = C + (n - 1) * step
        dense = wl.dense_mask(rng, w.Sq, cols, q_offset=0 if c["reuse"] else w.q_pos_base,
                              window=int(rng.integers(8, 200)), n_global=int(rng.integers(0, 8)), block=64)
    say(f"random ring {seed}: {c}")
    d = ram.Desc(B=w.B, Sq=w.Sq, Skv=C, H=w.H, Hkv=w.Hkv, D=w.D,
                 dtype=ram.RAM_BF16 if w.dtype == "bf16" else ram.RAM_F32, scale=w.scale,
                 softcap=w.softcap or 0.0, causal=w.causal)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)
    src = ram.MaskSrc(q_pos=t(w.q_pos), kv_pos=t(w.kv_pos), q_seg=t(w.q_seg), kv_seg=t(w.kv_seg),
                      dense=None if dense is None else torch.from_numpy(dense).to(DEV), dense_chunk_step=step)
    out = torch.full((w.B, w.Sq, w.H, w.D), float("nan"), device=DEV).to(w.q.dtype)
    lse = torch.full((w.B, w.H, w.Sq), float("nan"), device=DEV)
    ws = torch.empty(max(1, ram.ring_attn_workspace_bytes(d, n, src)), dtype=torch.uint8, device=DEV)
    sinks = None if w.sinks is None else w.sinks.to(DEV)
    ram.ring_attn_fwd_1gpu(d, n, r, w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), src, sinks, out, lse, ws)
    torch.cuda.synchronize()
    q, k, v, s64 = w.as_f64()
    qp, kp = w.positions()
    order = [(r - i) % n for i in range(n)] if r >= 0 else list(range(n))
    ro, rl = oracle.chunked(q, k, v, scale=w.scale, q_pos=qp, kv_pos=kp, bounds=[(i * C, (i + 1) * C) for i in range(n)],
                            order=order, q_seg=w.q_seg, kv_seg=w.kv_seg, causal=w.causal, softcap=w.softcap,
                            sinks=s64, dense=dense, dense_col0=None if dense is None else [i * step for i in range(n)])
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, w.dtype, f"random ring {seed}")


# ------------------------------------------------------------------------------ backward
N_BWD_CASES = 30


@pytest.mark.parametrize("seed", list(range(N_BWD_CASES)))
def test_random_ring_backward(seed):
    """ring_attn_bwd_1gpu on seeded random small rings (the forward's feature mix at smaller sizes)
    against oracle.chunked_bwd: dq, dk, dv at max error / max |ref|, dsinks against the sum of its
    terms' magnitudes, at the backward tolerances."""
    check_ring_backward(seed, _case(5000 + seed))


def check_ring_backward(seed: int, c: dict):
    """One random ring backward against the oracle."""
    from test_gpu_backward import GRAD_TOL, GRAD_TOL_F32, SINK_TOL, _rel, _sinks_check
    c = dict(c)
    c["Sq"] = min(c["Sq"], 400)
    c["chunk"] = min(c["chunk"], 300)
    if c["feature"] == "docs":
        c["Sq"] = c["chunk"] * c["n"]
    docs = (16, max(32, c["Sq"] // 2), 0.05) if c["feature"] == "docs" else None
    w = wl.make(f"randb{seed}", B=c["B"], H=c["H"], Hkv=c["Hkv"], Sq=c["Sq"], chunk=c["chunk"], n_chunks=c["n"],
                D=c["D"], dtype=c["dtype"], causal=c["causal"], softcap=c["cap"], with_sinks=c["sinks"],
                q_shard=c["q_shard"], docs=docs, seed=20_000 + seed)
    C, n, r = c["chunk"], c["n"], c["q_shard"]
    dense, step = None, 0
    if c["feature"] == "dense":
        rng = np.random.default_rng(95_000 + seed)
        step = 0 if c["reuse"] else C
        cols = C + (n - 1) * step
        dense = wl.dense_mask(rng, w.Sq, cols, q_offset=0 if c["reuse"] else w.q_pos_base,
                              window=int(rng.integers(8, 200)), n_global=int(rng.integers(0, 8)), block=64)
    say(f"random ring backward {seed}: {c}")
    d = ram.Desc(B=w.B, Sq=w.Sq, Skv=C, H=w.H, Hkv=w.Hkv, D=w.D,
                 dtype=ram.RAM_BF16 if w.dtype == "bf16" else ram.RAM_F32, scale=w.scale,
                 softcap=w.softcap or 0.0, causal=w.causal)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)
    src = ram.MaskSrc(q_pos=t(w.q_pos), kv_pos=t(w.kv_pos), q_seg=t(w.q_seg), kv_seg=t(w.kv_seg),
                      dense=None if dense is None else torch.from_numpy(dense).to(DEV), dense_chunk_step=step)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    sinks = None if w.sinks is None else w.sinks.to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.Sq, device=DEV)
    ws = torch.empty(max(1, ram.ring_attn_workspace_bytes(d, n, src)), dtype=torch.uint8, device=DEV)
    ram.ring_attn_fwd_1gpu(d, n, r, q, k, v, src, sinks, out, lse, ws)
    dout = torch.from_numpy(np.random.default_rng(30_000 + seed).standard_normal(
        (w.B, w.Sq, w.H, w.D)).astype(np.float32)).to(w.q.dtype)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    dsinks = None if sinks is None else torch.full((w.H,), float("nan"), device=DEV)
    wsb = torch.empty(max(1, ram.ring_attn_bwd_workspace_bytes(d, n, src)), dtype=torch.uint8, device=DEV)
    ram.ring_attn_bwd_1gpu(d, n, r, q, k, v, out, lse, dout.to(DEV), src, sinks, dq, dk, dv, dsinks, wsb)
    torch.cuda.synchronize()
    q64, k64, v64, s64 = w.as_f64()
    qp, kp = w.positions()
    kw = dict(scale=w.scale, q_pos=qp, kv_pos=kp, q_seg=w.q_seg, kv_seg=w.kv_seg, causal=w.causal,
              softcap=w.softcap, sinks=s64, dense=dense,
              dense_col0=None if dense is None else [i * step for i in range(n)])
    rq, rk, rv, rs = oracle.chunked_bwd(q64, k64, v64, dout.double().numpy(),
                                        bounds=[(i * C, (i + 1) * C) for i in range(n)], **kw)
    tol = GRAD_TOL_F32 if w.dtype == "f32" else GRAD_TOL
    what = f"random ring backward {seed}"
    for nm, g, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _rel(nm, g.float().cpu().numpy(), ref, tol, what)
    if sinks is not None:
        order = [(r - i) % n for i in range(n)] if r >= 0 else list(range(n))
        ro, rl = oracle.chunked(q64, k64, v64, bounds=[(i * C, (i + 1) * C) for i in range(n)], order=order, **kw)
        _sinks_check(dsinks.cpu().numpy(), rs, ro, rl, dout.double().numpy(), s64, what,
                     GRAD_TOL_F32 if w.dtype == "f32" else SINK_TOL)


# ------------------------------------------------------------------------------ block masks
N_MASK_CASES = 60
POISON = 0x5A5A5A5A


@pytest.mark.parametrize("seed", list(range(N_MASK_CASES)))
def test_random_block_mask_bitexact(seed):
    """build_block_mask on seeded random inputs: tile sizes in [16, 512], ragged lengths,
    sequential positions with offsets, shuffled positions or packed documents, random segment
    IDs with padding, causal or not, with or without a dense mask and tile bits. Classes, row
    counts, lists and the bits of PARTIAL tiles must equal oracle.block_mask / oracle.partial_bits
    bit for bit, and no bits may be written outside PARTIAL tiles."""
    rng = np.random.default_rng(110_000 + seed)
    B = int(rng.integers(1, 3))
    Sq, Skv = int(rng.integers(1, 1500)), int(rng.integers(1, 1500))
    bq, bk = int(rng.integers(16, 513)), int(rng.integers(16, 513))
    causal = bool(rng.random() < 0.7)
    kind = str(rng.choice(["seq", "shuffle", "docs", "segs"]))
    with_dense = bool(rng.random() < 0.4)
    with_bits = with_dense or bool(rng.random() < 0.5)
    qb = kb = 0
    qp = kp = qs = ks = None
    if kind == "seq":
        qb, kb = int(rng.integers(-500, 3000)), int(rng.integers(0, 3000))
    elif kind == "shuffle":
        qp = rng.integers(0, 2000, size=(B, Sq)).astype(np.int32)
        kp = rng.integers(0, 2000, size=(B, Skv)).astype(np.int32)
    elif kind == "docs":
        Skv = Sq
        qs, qp, _ = wl.packed_documents(rng, B, Sq, 8, max(16, Sq // 3), 0.05)
        ks, kp = qs, qp
    else:
        qs = rng.integers(-1, 4, size=(B, Sq)).astype(np.int32)
        ks = rng.integers(-1, 4, size=(B, Skv)).astype(np.int32)
    dense = None
    if with_dense:
        dense = wl.dense_mask(rng, Sq, Skv, q_offset=qb - kb, window=int(rng.integers(4, 300)),
                              n_global=int(rng.integers(0, 20)), block=int(rng.integers(16, 200)))
    say(f"random block mask {seed}: B={B} Sq={Sq} Skv={Skv} tile={bq}x{bk} causal={causal} {kind} "
        f"dense={with_dense} bits={with_bits} q_base={qb} kv_base={kb}")
    d = ram.Desc(B=B, Sq=Sq, Skv=Skv, H=1, Hkv=1, D=128, causal=causal, block_q=bq, block_kv=bk)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)
    src = ram.MaskSrc(q_pos=t(qp), kv_pos=t(kp), q_seg=t(qs), kv_seg=t(ks), q_pos_base=qb, kv_pos_base=kb,
                      dense=None if dense is None else torch.from_numpy(dense).to(DEV))
    bm = ram.alloc_block_mask(d, with_bits=with_bits)
    bm.tile_class.fill_(0xAB)
    bm.row_cnt.fill_(-7)
    bm.col_idx.fill_(-7)
    if with_bits:
        bm.bits.fill_(POISON)
    ram.build_block_mask(d, src, bm)
    torch.cuda.synchronize()
    nQb, nKb, W = bm.nQb, bm.nKb, -(-bk // 32)
    cls = bm.tile_class.cpu().numpy()[: B * nQb * nKb].reshape(B, nQb, nKb)
    cnt = bm.row_cnt.cpu().numpy()[: B * nQb].reshape(B, nQb)
    col = bm.col_idx.cpu().numpy()[: B * nQb * nKb].reshape(B, nQb, nKb)
    if with_bits:
        bits = bm.bits.cpu().numpy().view(np.uint32)[: B * nQb * nKb * bq * W].reshape(B, nQb, nKb, bq, W)
    for b in range(B):
        qpb = qp[b] if qp is not None else qb + np.arange(Sq)
        kpb = kp[b] if kp is not None else kb + np.arange(Skv)
        ok = oracle.allowed(qpb, kpb, None if qs is None else qs[b], None if ks is None else ks[b], causal,
                            dense=dense)
        rc, rn, ri = oracle.block_mask(ok, bq, bk)
        assert np.array_equal(cls[b], rc), f"classes differ (b={b})"
        assert np.array_equal(cnt[b], rn), f"row counts differ (b={b})"
        assert np.array_equal(col[b], ri), f"tile lists differ (b={b})"
        if with_bits:
            rb = oracle.partial_bits(ok, bq, bk)
            part = rc == oracle.TILE_PARTIAL
            assert np.array_equal(bits[b][part], rb[part]), f"PARTIAL tile bits differ (b={b})"
            assert np.all(bits[b][~part] == POISON), f"bits written outside PARTIAL tiles (b={b})"
