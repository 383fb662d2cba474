"""GPU parity of the backward (dq, dk, dv, dsinks) against the float64 oracle.

The GPU forward supplies out and lse to the GPU backward, as a caller would;
the oracle computes its own forward and gradients in float64 from the same
rounded inputs (oracle.attention_bwd / oracle.chunked_bwd). Tolerance: bf16
inputs, normalised max error max|gpu - ref| / max|ref| <= 2e-2 for dq, dk, dv
(P and dS enter the matrix cores in bf16, 2^-9 relative each, and the ring's
outputs are bf16) and <= 1e-2 for dsinks (float32 sums of rounded D terms).
Transposed tile lists are compared bit for bit with the transpose of the
oracle's classes.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import ring_attention_merge_amd as ram
from ring_attention_merge_amd import workloads as wl
from gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"
GRAD_TOL = 2e-2
GRAD_TOL_F32 = 1e-5   # float32 inputs: float32 rounding over a few thousand terms is ~1e-6
SINK_TOL = 1e-2   # dsinks error over sum_i exp(sink - lse_i) |D_i| (see _sinks_check)


def _i32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def _rel(name, got, ref, tol, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what} {name}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{what} {name}: non-finite values"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    rel = err / scale if scale > 0 else err
    say(f"{what} {name}: max err {err:.3e}, max |ref| {scale:.3e}, normalised {rel:.3e} (tol {tol:.0e})")
    assert rel <= tol, f"{what} {name}: normalised error {rel:.3e} > {tol}"


def _sinks_check(got, ref, out, lse, dout, sinks, what, tol=SINK_TOL):
    """dsinks_h = -sum_i w_i D_i (w_i = exp(sink_h - lse_i), D_i = dout_i . out_i) is a signed
    sum that can cancel to far below its terms, so its error is measured against the sum of the
    terms' magnitudes, sum_i w_i |D_i|, from the oracle's float64 out and lse. Per term the
    backward carries the forward's lse error (1e-3 absolute, so 1e-3 relative in w_i) and the
    bf16 rounding of out inside D_i (about 2^-8), about 5e-3 together: the bound is 1e-2."""
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{what} dsinks: non-finite values"
    Dv = np.einsum("bihd,bihd->bhi", dout, out)
    wts = np.where(np.isfinite(lse), np.exp(np.asarray(sinks)[None, :, None] - lse), 0.0)
    mag = (wts * np.abs(Dv)).sum(axis=(0, 2))
    err = np.abs(got - ref)
    rel = float(np.max(err / np.maximum(mag, 1e-30)))
    say(f"{what} dsinks: max err {float(err.max()):.3e}, max |ref| {float(np.abs(ref).max()):.3e}, "
        f"err / sum w|D| {rel:.3e} (tol {tol:.0e})")
    assert rel <= tol, f"{what} dsinks: error {rel:.3e} of sum w|D| > {tol}"


# ------------------------------------------------------------------------------ transposed lists
@pytest.mark.parametrize("case", ["causal_ragged", "docs", "dense"])
def test_col_lists_bitexact(case):
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    B, Sq, Skv, causal, qb = 2, 700, 520, True, 300
    qp = kp = qs = ks = dense = None
    if case == "docs":
        Sq = Skv = 900
        qb = 0
        qs, qp, _ = wl.packed_documents(rng, B, Sq, 30, 300, 0.05)
        ks, kp = qs, qp
    if case == "dense":
        dense = wl.dense_mask(rng, Sq, Skv, q_offset=qb, window=100, n_global=8, block=64)
    d = ram.Desc(B=B, Sq=Sq, Skv=Skv, H=1, Hkv=1, D=128, causal=causal)
    src = ram.MaskSrc(q_pos=_i32(qp), kv_pos=_i32(kp), q_seg=_i32(qs), kv_seg=_i32(ks), q_pos_base=qb,
                      dense=None if dense is None else torch.from_numpy(dense).to(DEV))
    bm = ram.alloc_block_mask(d, with_bits=dense is not None, with_cols=True)
    bm.col_cnt.fill_(-7)
    bm.row_idx.fill_(-7)
    say(f"transposed lists {case}")
    ram.build_block_mask(d, src, bm)
    torch.cuda.synchronize()
    nQb, nKb = bm.nQb, bm.nKb
    cc = bm.col_cnt.cpu().numpy()[: B * nKb].reshape(B, nKb)
    ri = bm.row_idx.cpu().numpy()[: B * nKb * nQb].reshape(B, nKb, nQb)
    for b in range(B):
        qpb = qp[b] if qp is not None else qb + np.arange(Sq)
        kpb = kp[b] if kp is not None else np.arange(Skv)
        ok = oracle.allowed(qpb, kpb, None if qs is None else qs[b], None if ks is None else ks[b], causal, dense)
        cls, _, _ = oracle.block_mask(ok, 128, 64)
        for kb in range(nKb):
            nz = np.nonzero(cls[:, kb])[0]
            assert cc[b, kb] == len(nz), f"count b={b} kb={kb}"
            assert np.array_equal(ri[b, kb, :len(nz)], nz) and np.all(ri[b, kb, len(nz):] == -1), f"list b={b} kb={kb}"


# ------------------------------------------------------------------------------ one chunk
CASES = {
    # name: B, Sq, Skv, H, Hkv, causal, q_base, extra, cap, sinks
    "causal_gqa": (1, 384, 384, 4, 2, True, 0, None, None, False),
    "ragged_offset_sinks": (2, 200, 333, 2, 1, True, 150, None, None, True),
    "noncausal_segs_cap_sinks": (1, 300, 270, 4, 4, False, 0, "segs", 5.0, True),
    "docs_cap": (2, 520, 520, 4, 2, True, 0, "docs", 30.0, False),
    "shuffled_pos": (1, 250, 300, 2, 2, True, 0, "shuffle", None, False),
    "empty_rows": (1, 260, 190, 2, 1, True, -70, None, None, False),
    "mqa": (1, 256, 512, 8, 1, True, 256, None, None, True),
    "dense_causal": (1, 300, 333, 4, 2, True, 40, "dense", None, False),
    "dense_noncausal_cap_sinks": (2, 257, 200, 2, 2, False, 0, "dense", 20.0, True),
    "tiny": (1, 1, 1, 1, 1, True, 0, None, None, False),
    # head dim 64 (eight 16-byte chunks per row: its own swizzle and DMA slabs)
    "d64_causal_gqa_sinks": (2, 300, 333, 4, 2, True, 40, None, None, True, 64),
    "d64_segs_cap": (1, 260, 300, 2, 2, False, 0, "segs", 10.0, False, 64),
    "d64_docs": (1, 384, 384, 2, 1, True, 0, "docs", None, False, 64),
    "d64_dense_cap_sinks": (1, 257, 270, 4, 4, True, 20, "dense", 30.0, True, 64),
    # float32 inputs (the exact-reference dtype)
    "f32_d64_causal": (1, 256, 256, 2, 2, True, 0, None, None, False, 64, "f32"),
    "f32_d128_gqa_segs_cap_sinks": (2, 200, 230, 4, 2, False, 0, "segs", 8.0, True, 128, "f32"),
    "f32_d64_dense_ragged": (1, 130, 200, 2, 1, True, 30, "dense", None, False, 64, "f32"),
}


def _inputs(name):
    B, Sq, Skv, H, Hkv, causal, qb, extra, cap, with_sinks = CASES[name][:10]
    D = CASES[name][10] if len(CASES[name]) > 10 else 128
    f32 = len(CASES[name]) > 11 and CASES[name][11] == "f32"
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.float32 if f32 else torch.bfloat16)
    q = bf(rng.standard_normal((B, Sq, H, D)))
    k = bf(rng.standard_normal((B, Skv, Hkv, D)))
    v = bf(rng.standard_normal((B, Skv, Hkv, D)))
    dout = bf(rng.standard_normal((B, Sq, H, D)))
    sinks = torch.from_numpy(rng.standard_normal(H).astype(np.float32)) if with_sinks else None
    qp = np.broadcast_to(qb + np.arange(Sq), (B, Sq)).astype(np.int32)
    kp = np.broadcast_to(np.arange(Skv), (B, Skv)).astype(np.int32)
    qs = ks = dense = None
    explicit = False
    if extra == "segs":
        qs = rng.integers(-1, 3, size=(B, Sq)).astype(np.int32)
        ks = rng.integers(-1, 3, size=(B, Skv)).astype(np.int32)
    elif extra == "docs":
        qs, qp, _ = wl.packed_documents(rng, B, Sq, 16, 200, 0.05)
        ks, kp = qs, qp
        explicit = True
    elif extra == "shuffle":
        qp = rng.integers(0, 300, size=(B, Sq)).astype(np.int32)
        kp = rng.integers(0, 300, size=(B, Skv)).astype(np.int32)
        explicit = True
    elif extra == "dense":
        dense = wl.dense_mask(rng, Sq, Skv, q_offset=qb, window=60, n_global=4, block=64)
    src = ram.MaskSrc(q_pos=_i32(qp) if explicit else None, kv_pos=_i32(kp) if explicit else None,
                      q_pos_base=0 if explicit else qb, q_seg=_i32(qs), kv_seg=_i32(ks),
                      dense=None if dense is None else torch.from_numpy(dense).to(DEV))
    d = ram.Desc(B=B, Sq=Sq, Skv=Skv, H=H, Hkv=Hkv, D=D, dtype=ram.RAM_F32 if f32 else ram.RAM_BF16,
                 scale=1.0 / math.sqrt(D), softcap=cap or 0.0, causal=causal)
    ref_kw = dict(scale=d.scale, q_pos=qp, kv_pos=kp, q_seg=qs, kv_seg=ks, causal=causal, softcap=cap, dense=dense,
                  sinks=None if sinks is None else sinks.double().numpy())
    return d, q, k, v, dout, sinks, src, ref_kw


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunk_backward(name):
    d, q, k, v, dout, sinks, src, ref_kw = _inputs(name)
    say(f"attn_bwd_chunk {name}: B={d.B} Sq={d.Sq} Skv={d.Skv} H={d.H}/{d.Hkv} D={d.D}")
    B, Sq, Skv, H, Hkv, D = d.B, d.Sq, d.Skv, d.H, d.Hkv, d.D
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV)
    sd = None if sinks is None else sinks.to(DEV)
    # forward through the library (one chunk, bf16 result)
    out = torch.full((B, Sq, H, D), float("nan"), device=DEV).to(q.dtype)
    lse = torch.full((B, H, Sq), float("nan"), device=DEV)
    ws = torch.empty(max(1, ram.ring_attn_workspace_bytes(d, 1, src)), dtype=torch.uint8, device=DEV)
    ram.ring_attn_fwd_1gpu(d, 1, -1, qd, kd, vd, src, sd, out, lse, ws)
    # backward of the chunk
    bm = ram.alloc_block_mask(d, with_bits=src.dense is not None, with_cols=True)
    ram.build_block_mask(d, src, bm)
    delta = torch.full((2, B, H, Sq), float("nan"), device=DEV)
    dsinks = None if sinks is None else torch.full((H,), float("nan"), device=DEV)
    ram.attn_bwd_prep(d, out, dod, lse, sd, delta, dsinks)
    # the prep's second row array: the forward's lse in base 2, +inf for rows with no key
    l32 = lse.cpu().numpy()
    want = np.where(np.isneginf(l32), np.float32(np.inf), l32 * np.float32(1.4426950408889634))
    got = delta[1].cpu().numpy()
    assert np.array_equal(np.isinf(got), np.isinf(want)) and np.allclose(got[np.isfinite(want)], want[np.isfinite(want)],
                                                                         rtol=1e-6, atol=0), name
    dq = torch.full((B, Sq, H, D), float("nan"), device=DEV)
    dk = torch.full((B, Skv, Hkv, D), float("nan"), device=DEV)
    dv = torch.full((B, Skv, Hkv, D), float("nan"), device=DEV)
    ram.attn_bwd_chunk(d, qd, kd, vd, dod, lse, delta, src, bm, ram.RAM_OUT_WRITE, dq, dk, dv)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = (x.double().numpy() for x in (q, k, v, dout))
    rq, rk, rv, rs = oracle.attention_bwd(q64, k64, v64, do64, **ref_kw)
    tol = GRAD_TOL_F32 if d.dtype == ram.RAM_F32 else GRAD_TOL
    _rel("dq", dq.cpu().numpy(), rq, tol, name)
    _rel("dk", dk.cpu().numpy(), rk, tol, name)
    _rel("dv", dv.cpu().numpy(), rv, tol, name)
    if sinks is not None:
        ro, rl = oracle.attention(q64, k64, v64, **ref_kw)
        _sinks_check(dsinks.cpu().numpy(), rs, ro, rl, do64, ref_kw["sinks"], name,
                     GRAD_TOL_F32 if d.dtype == ram.RAM_F32 else SINK_TOL)


def test_chunk_backward_add_mode():
    """dq_mode MERGE adds the chunk's dq to what is there: two calls = twice one call."""
    d, q, k, v, dout, sinks, src, _ = _inputs("causal_gqa")
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV)
    out = torch.empty_like(qd)
    lse = torch.empty(d.B, d.H, d.Sq, device=DEV)
    ws = torch.empty(ram.ring_attn_workspace_bytes(d, 1, src), dtype=torch.uint8, device=DEV)
    ram.ring_attn_fwd_1gpu(d, 1, -1, qd, kd, vd, src, None, out, lse, ws)
    bm = ram.alloc_block_mask(d, with_cols=True)
    ram.build_block_mask(d, src, bm)
    delta = torch.empty(2, d.B, d.H, d.Sq, device=DEV)
    ram.attn_bwd_prep(d, out, dod, lse, None, delta, None)
    dq1 = torch.empty(d.B, d.Sq, d.H, 128, device=DEV)
    dq2 = torch.empty_like(dq1)
    dk = torch.empty(d.B, d.Skv, d.Hkv, 128, device=DEV)
    dv = torch.empty_like(dk)
    ram.attn_bwd_chunk(d, qd, kd, vd, dod, lse, delta, src, bm, ram.RAM_OUT_WRITE, dq1, dk, dv)
    ram.attn_bwd_chunk(d, qd, kd, vd, dod, lse, delta, src, bm, ram.RAM_OUT_WRITE, dq2, dk, dv)
    ram.attn_bwd_chunk(d, qd, kd, vd, dod, lse, delta, src, bm, ram.RAM_OUT_MERGE, dq2, dk, dv)
    torch.cuda.synchronize()
    assert torch.equal(dq2, dq1 * 2)


# ------------------------------------------------------------------------------ ring
RING = {
    "shard3of4": lambda: wl.c2_ring_shard(Sq=256, H=2, seed=31),
    "shard1of3_ragged_gqa": lambda: wl.make("b1", B=2, H=4, Hkv=2, Sq=200, chunk=200, n_chunks=3, D=128,
                                            q_shard=1, seed=32),
    "docs": lambda: wl.c3_packed_docs(S=1024, B=2, H=2, len_lo=32, len_hi=256, seed=33),
    # documents across three chunks: the dq ring masks every visit from the chunk's positions and
    # segment IDs (tile bits)
    "docs_3chunks_gqa": lambda: wl.make("rd128", B=2, H=4, Hkv=2, Sq=768, chunk=256, n_chunks=3, D=128,
                                        docs=(32, 200, 0.05), seed=43),
    "gqa_cap_sinks": lambda: wl.c4_gqa_cap_sinks(S=1024, H=8, Hkv=2, seed=34),
    "mqa_cap_sinks": lambda: wl.c4_gqa_cap_sinks(S=768, H=4, Hkv=1, seed=35),
    # 16 heads on one kv head, 4 kv tiles per chunk: the dk / dv launch splits the group's heads
    # over 16 workgroups and adds their partial sums
    "mqa16_ragged": lambda: wl.make("mq16", B=1, H=16, Hkv=1, Sq=250, chunk=250, n_chunks=2, D=128, seed=42),
    "noncausal_sinks": lambda: wl.make("nc", B=1, H=2, Hkv=2, Sq=100, chunk=70, n_chunks=3, D=128, causal=False,
                                       seed=36, with_sinks=True),
    "d64_shard2of4_gqa_cap_sinks": lambda: wl.make("r64", B=2, H=4, Hkv=2, Sq=320, chunk=320, n_chunks=4, D=64,
                                                   q_shard=2, softcap=20.0, with_sinks=True, seed=38),
    "d64_docs": lambda: wl.make("r64d", B=1, H=2, Hkv=1, Sq=768, chunk=256, n_chunks=3, D=64, docs=(32, 200, 0.05),
                                seed=39),
    "f32_c1_shape": lambda: wl.make("rf32", B=1, H=2, Hkv=2, Sq=256, chunk=128, n_chunks=2, D=64, dtype="f32",
                                    seed=40),
    "f32_shard1of3_gqa_cap_sinks": lambda: wl.make("rf32s", B=2, H=4, Hkv=2, Sq=150, chunk=150, n_chunks=3, D=128,
                                                   dtype="f32", q_shard=1, softcap=10.0, with_sinks=True, seed=41),
}


def _run_ring_bwd(w, dout, src=None):
    d = ram.Desc(B=w.B, Sq=w.Sq, Skv=w.chunk, H=w.H, Hkv=w.Hkv, D=w.D,
                 dtype=ram.RAM_F32 if w.dtype == "f32" else ram.RAM_BF16, scale=w.scale, softcap=w.softcap or 0.0,
                 causal=w.causal)
    if src is None:
        src = ram.MaskSrc(q_pos=_i32(w.q_pos), kv_pos=_i32(w.kv_pos), q_seg=_i32(w.q_seg), kv_seg=_i32(w.kv_seg))
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    sinks = None if w.sinks is None else w.sinks.to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.Sq, device=DEV)
    ws = torch.empty(max(1, ram.ring_attn_workspace_bytes(d, w.n_chunks, src)), dtype=torch.uint8, device=DEV)
    ram.ring_attn_fwd_1gpu(d, w.n_chunks, w.q_shard, q, k, v, src, sinks, out, lse, ws)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    dsinks = None if sinks is None else torch.full((w.H,), float("nan"), device=DEV)
    wsb = torch.empty(max(1, ram.ring_attn_bwd_workspace_bytes(d, w.n_chunks, src)), dtype=torch.uint8, device=DEV)
    ram.ring_attn_bwd_1gpu(d, w.n_chunks, w.q_shard, q, k, v, out, lse, dout.to(DEV), src, sinks, dq, dk, dv,
                           dsinks, wsb)
    torch.cuda.synchronize()
    return dq.float().cpu().numpy(), dk.float().cpu().numpy(), dv.float().cpu().numpy(), \
        None if dsinks is None else dsinks.cpu().numpy()


def _ring_ref(w, dout, dense=None, dense_col0=None):
    q, k, v, s64 = w.as_f64()
    qp, kp = w.positions()
    bounds = [(c * w.chunk, (c + 1) * w.chunk) for c in range(w.n_chunks)]
    return oracle.chunked_bwd(q, k, v, dout.double().numpy(), scale=w.scale, q_pos=qp, kv_pos=kp, bounds=bounds,
                              q_seg=w.q_seg, kv_seg=w.kv_seg, causal=w.causal, softcap=w.softcap, sinks=s64,
                              dense=dense, dense_col0=dense_col0)


def _ring_sinks_check(w, dout, got, ref, what, dense=None):
    tol = GRAD_TOL_F32 if w.dtype == "f32" else SINK_TOL
    q, k, v, s64 = w.as_f64()
    qp, kp = w.positions()
    ro, rl = oracle.attention(q, k, v, scale=w.scale, q_pos=qp, kv_pos=kp, q_seg=w.q_seg, kv_seg=w.kv_seg,
                              causal=w.causal, softcap=w.softcap, sinks=s64, dense=dense)
    _sinks_check(got, ref, ro, rl, dout.double().numpy(), s64, what, tol)


@pytest.mark.parametrize("name", sorted(RING))
def test_ring_backward(name):
    w = RING[name]()
    dout = torch.from_numpy(np.random.default_rng(zlib.crc32(name.encode())).standard_normal(
        (w.B, w.Sq, w.H, w.D)).astype(np.float32)).to(w.q.dtype)
    say(f"ring_attn_bwd_1gpu {name}: B={w.B} H={w.H}/{w.Hkv} Sq={w.Sq} chunks={w.n_chunks}x{w.chunk}")
    got = _run_ring_bwd(w, dout)
    ref = _ring_ref(w, dout)
    for nm, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        _rel(nm, g, r, GRAD_TOL_F32 if w.dtype == "f32" else GRAD_TOL, name)
    if w.sinks is not None:
        _ring_sinks_check(w, dout, got[3], ref[3], name)


def test_ring_backward_dense_global():
    w = wl.make("bd", B=1, H=4, Hkv=2, Sq=256, chunk=192, n_chunks=3, D=128, q_shard=2, seed=37, with_sinks=True)
    rng = np.random.default_rng(37)
    dense = wl.dense_mask(rng, w.Sq, w.Skv, q_offset=w.q_pos_base, window=80, n_global=5, block=64)
    src = ram.MaskSrc(dense=torch.from_numpy(dense).to(DEV), dense_chunk_step=w.chunk)
    dout = torch.from_numpy(rng.standard_normal((w.B, w.Sq, w.H, w.D)).astype(np.float32)).to(torch.bfloat16)
    say("ring_attn_bwd_1gpu dense global")
    got = _run_ring_bwd(w, dout, src)
    ref = _ring_ref(w, dout, dense=dense)
    for nm, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        _rel(nm, g, r, GRAD_TOL, "dense global")
    _ring_sinks_check(w, dout, got[3], ref[3], "dense global", dense=dense)


def test_ring_backward_c2_full():
    """The 4-step ring shard at full size (local Sq 4096 as shard 3 of 4, 4 chunks of 4096, H=8, D=128):
    every element of dq, dk, dv against the oracle."""
    w = wl.c2_ring_shard()
    dout = torch.from_numpy(np.random.default_rng(2003).standard_normal(
        (w.B, w.Sq, w.H, w.D)).astype(np.float32)).to(torch.bfloat16)
    say(f"ring_attn_bwd_1gpu {w.name} (full)")
    got = _run_ring_bwd(w, dout)
    ref = _ring_ref(w, dout)
    for nm, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        _rel(nm, g, r, GRAD_TOL, "c2 full")


FULL_SIZE_BWD = {
    "c5": wl.c5_long_causal,
    "c4_gqa_cap_sinks": wl.c4_gqa_cap_sinks,
    "c4_mqa_cap_sinks": lambda: wl.c4_gqa_cap_sinks(Hkv=1),
}


@pytest.mark.parametrize("name", list(FULL_SIZE_BWD))
def test_ring_backward_full_size_sampled(name):
    """The 32k causal ring that bench.py --backward times (B 1, H 32 / Hkv 8, Sq = Skv = 32768 in 8
    chunks of 4096, D 128, bf16) and the soft-cap GQA / MQA rings with sinks (16384 keys in 4
    chunks), at full size, against the oracle where it computes row by row:
    - dq at sampled query rows (edge rows of every chunk and seeded ones, every head), from
      oracle.attention_dq, which needs only those rows and every key;
    - dk and dv at the last 128 keys: under the causal mask only the last 128 query rows attend
      them, so oracle.attention_bwd over those rows (against every key) gives them exactly;
    - without sinks, an identity of the exact gradient over every key: within each KV head the
      dv rows sum to the dout rows of all query rows and heads sharing it (each row's weights
      sum to one, and every row here has an allowed key). Each GPU dv row is a bf16 value of
      float32 sums of bf16 weights times dout, within 2^-8 of its exact value relative to its
      terms' magnitudes, so the bound is 2^-8 of sum_j |dv_j| per element (plus float64
      summation)."""
    w = FULL_SIZE_BWD[name]()
    dout = torch.from_numpy(np.random.default_rng(2005).standard_normal(
        (w.B, w.Sq, w.H, w.D)).astype(np.float32)).to(torch.bfloat16)
    say(f"ring_attn_bwd_1gpu {w.name} (full size, sampled rows and keys)")
    dq, dk, dv, _ = _run_ring_bwd(w, dout)
    q64, k64, v64, s64 = w.as_f64()
    do64 = dout.double().numpy()
    qp, kp = w.positions()
    kw = dict(scale=w.scale, kv_pos=kp, causal=True, softcap=w.softcap, sinks=s64)
    rows = wl.sampled_rows(w.Sq, w.chunk, n=24, seed=2006)
    ref_dq = oracle.attention_dq(q64[:, rows], k64, v64, do64[:, rows], q_pos=qp[:, rows], **kw)
    _rel("dq", dq[:, rows], ref_dq, GRAD_TOL, f"{name} full, {len(rows)} sampled rows")
    tail = 128
    r0 = w.Sq - tail
    _, rdk, rdv, _ = oracle.attention_bwd(q64[:, r0:], k64, v64, do64[:, r0:], q_pos=qp[:, r0:], **kw)
    _rel("dk", dk[:, r0:], rdk[:, r0:], GRAD_TOL, f"{name} full, last {tail} keys")
    _rel("dv", dv[:, r0:], rdv[:, r0:], GRAD_TOL, f"{name} full, last {tail} keys")
    if s64 is None:
        G = w.H // w.Hkv
        lhs = dv.astype(np.float64).sum(axis=1)                                        # [B, Hkv, D]
        rhs = do64.reshape(w.B, w.Sq, w.Hkv, G, w.D).sum(axis=(1, 3))                  # [B, Hkv, D]
        bound = 2.0 ** -8 * np.abs(dv.astype(np.float64)).sum(axis=1) + 1e-9 * np.abs(rhs)
        worst = float(np.max(np.abs(lhs - rhs) / bound))
        say(f"{name} full: sum_j dv_j vs sum of dout over rows and heads: max |diff| "
            f"{float(np.abs(lhs - rhs).max()):.3e}, at most {worst:.3f} of the rounding bound")
        assert worst <= 1.0, f"{name} full: sum_j dv_j departs from the summed dout ({worst:.3f} of the bound)"


def test_backward_deterministic():
    w = RING["gqa_cap_sinks"]()
    dout = torch.from_numpy(np.random.default_rng(9).standard_normal((w.B, w.Sq, w.H, w.D)).astype(np.float32)).to(
        torch.bfloat16)
    a = _run_ring_bwd(w, dout)
    b = _run_ring_bwd(w, dout)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
