"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances (written in gpu_util): out max-abs <= 2e-2 for bf16 inputs and
<= 1e-4 for fp32, lse <= 1e-3, rows with no allowed key exactly (0, -inf),
block-mask classes and lists bit-exact. Outputs are poisoned with NaN before
each call so unwritten elements fail.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import ring_attention_merge_amd as ram
from ring_attention_merge_amd import workloads as wl
from gpu_util import OUT_TOL, compare, mask_src, oracle_ref, ring_by_chunks, ring_desc, ring_splits, run_ring, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _i32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


# ------------------------------------------------------------------------------ block mask
MASK_CASES = {
    "seq_causal_ragged": dict(B=1, Sq=300, Skv=200, qb=150, kb=0),
    "seq_causal_ring_shard": dict(B=1, Sq=4096, Skv=4096, qb=3 * 4096, kb=2 * 4096),
    "seq_causal_diag": dict(B=2, Sq=4096, Skv=4096, qb=0, kb=0),
    "seq_noncausal": dict(B=1, Sq=77, Skv=129, qb=0, kb=0, causal=False),
    "pos_shuffled": dict(B=2, Sq=333, Skv=271, pos="shuffle"),
    "docs_pad": dict(B=2, Sq=1000, Skv=1000, docs=True),
    "docs_pad_noncausal": dict(B=1, Sq=700, Skv=700, docs=True, causal=False),
    "segments_random": dict(B=1, Sq=257, Skv=190, segs="random"),
}
TILES = [(128, 64), (128, 128), (64, 32), (16, 16), (256, 512), (48, 80)]


def _mask_case(name):
    c = MASK_CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    B, Sq, Skv = c["B"], c["Sq"], c["Skv"]
    causal = c.get("causal", True)
    qp = kp = qs = ks = None
    qb, kb = c.get("qb", 0), c.get("kb", 0)
    if c.get("pos") == "shuffle":
        qp = rng.integers(0, 400, size=(B, Sq)).astype(np.int32)
        kp = rng.integers(0, 400, size=(B, Skv)).astype(np.int32)
    if c.get("docs"):
        seg, pos, _ = wl.packed_documents(rng, B, Sq, 20, 300, 0.05)
        qs = ks = seg
        qp = kp = pos
    if c.get("segs") == "random":
        qs = rng.integers(-1, 3, size=(B, Sq)).astype(np.int32)
        ks = rng.integers(-1, 3, size=(B, Skv)).astype(np.int32)
    return B, Sq, Skv, causal, qp, kp, qs, ks, qb, kb


@pytest.mark.parametrize("tile", TILES, ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("name", sorted(MASK_CASES))
def test_block_mask_bitexact(name, tile):
    B, Sq, Skv, causal, qp, kp, qs, ks, qb, kb = _mask_case(name)
    say(f"block mask {name} tile {tile}")
    d = ram.Desc(B=B, Sq=Sq, Skv=Skv, H=1, Hkv=1, D=128, causal=causal, block_q=tile[0], block_kv=tile[1])
    src = ram.MaskSrc(q_pos=_i32(qp), kv_pos=_i32(kp), q_seg=_i32(qs), kv_seg=_i32(ks), q_pos_base=qb,
                      kv_pos_base=kb)
    bm = ram.alloc_block_mask(d)
    bm.tile_class.fill_(0xAB)
    bm.row_cnt.fill_(-7)
    bm.col_idx.fill_(-7)
    ram.build_block_mask(d, src, bm)
    torch.cuda.synchronize()
    nQb, nKb = bm.nQb, bm.nKb
    cls = bm.tile_class.cpu().numpy()[: B * nQb * nKb].reshape(B, nQb, nKb)
    cnt = bm.row_cnt.cpu().numpy()[: B * nQb].reshape(B, nQb)
    col = bm.col_idx.cpu().numpy()[: B * nQb * nKb].reshape(B, nQb, nKb)
    for b in range(B):
        qpb = qp[b] if qp is not None else qb + np.arange(Sq)
        kpb = kp[b] if kp is not None else kb + np.arange(Skv)
        ok = oracle.allowed(qpb, kpb, None if qs is None else qs[b], None if ks is None else ks[b], causal)
        rc, rn, ri = oracle.block_mask(ok, tile[0], tile[1])
        assert np.array_equal(cls[b], rc), f"classes differ (b={b})"
        assert np.array_equal(cnt[b], rn), f"row counts differ (b={b})"
        assert np.array_equal(col[b], ri), f"tile lists differ (b={b})"


# ------------------------------------------------------------------------------ one chunk
def _chunk_ref(q, k, v, scale, qp, kp, qs, ks, causal, cap, sinks):
    return oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale=scale,
                            q_pos=qp, kv_pos=kp, q_seg=qs, kv_seg=ks, causal=causal, softcap=cap,
                            sinks=None if sinks is None else sinks.double().numpy())


def _run_chunk(d, q, k, v, src, sinks, mode, out, lse):
    bq, bk = ram.kernel_tile(d.dtype, d.D)
    dm = ram.Desc(**{**d.__dict__, "block_q": bq, "block_kv": bk})
    bm = ram.alloc_block_mask(dm, with_bits=True)
    ram.build_block_mask(dm, src, bm)
    ram.attn_fwd_chunk(dm, q, k, v, src, bm, sinks, mode, out, lse)


CHUNK_CASES = {
    # name: dtype, D, B, Sq, Skv, H, Hkv, causal, q_base, positions, segments, cap, sinks
    "bf16_d128_causal_gqa": ("bf16", 128, 1, 384, 384, 4, 2, True, 0, "seq", False, None, False),
    "bf16_d128_ragged": ("bf16", 128, 2, 200, 333, 2, 2, True, 150, "seq", False, None, False),
    "bf16_d128_empty_rows": ("bf16", 128, 1, 260, 190, 2, 1, True, -70, "seq", False, None, True),
    "bf16_d128_shuffled_pos": ("bf16", 128, 1, 250, 300, 2, 2, True, 0, "shuffle", False, None, False),
    "bf16_d128_docs_cap_sinks": ("bf16", 128, 2, 520, 520, 4, 2, True, 0, "docs", True, 50.0, True),
    "bf16_d64_noncausal_segs_cap": ("bf16", 64, 1, 300, 270, 4, 4, False, 0, "seq", True, 5.0, True),
    "bf16_d128_mqa": ("bf16", 128, 1, 256, 512, 8, 1, True, 256, "seq", False, None, False),
    "bf16_d128_tiny": ("bf16", 128, 1, 1, 1, 1, 1, True, 0, "seq", False, None, False),
    "f32_d64_causal": ("f32", 64, 1, 256, 256, 2, 2, True, 0, "seq", False, None, False),
    "f32_d128_segs_cap_sinks": ("f32", 128, 1, 333, 333, 4, 2, True, 0, "docs", True, 3.0, True),
    "f32_d64_ragged_gqa": ("f32", 64, 2, 131, 77, 6, 3, True, 40, "seq", False, None, False),
}


def _make_chunk_inputs(name):
    dt, D, B, Sq, Skv, H, Hkv, causal, qb, pos, segs, cap, with_sinks = CHUNK_CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    q = torch.from_numpy(rng.standard_normal((B, Sq, H, D), dtype=np.float32)).to(tdt)
    k = torch.from_numpy(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32)).to(tdt)
    v = torch.from_numpy(rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32)).to(tdt)
    sinks = torch.from_numpy(rng.standard_normal(H, dtype=np.float32)) if with_sinks else None
    qp = np.broadcast_to(qb + np.arange(Sq), (B, Sq)).astype(np.int32)
    kp = np.broadcast_to(np.arange(Skv), (B, Skv)).astype(np.int32)
    qs = ks = None
    explicit = False
    if pos == "shuffle":
        qp = rng.integers(0, 300, size=(B, Sq)).astype(np.int32)
        kp = rng.integers(0, 300, size=(B, Skv)).astype(np.int32)
        explicit = True
    if pos == "docs":
        assert Sq == Skv
        seg, p, _ = wl.packed_documents(rng, B, Sq, 16, 200, 0.05)
        qp = kp = p
        qs = ks = seg
        explicit = True
    elif segs:
        qs = rng.integers(-1, 4, size=(B, Sq)).astype(np.int32)
        ks = rng.integers(-1, 4, size=(B, Skv)).astype(np.int32)
    src = ram.MaskSrc(q_pos=_i32(qp) if explicit else None, kv_pos=_i32(kp) if explicit else None,
                      q_pos_base=0 if explicit else qb, q_seg=_i32(qs), kv_seg=_i32(ks))
    d = ram.Desc(B=B, Sq=Sq, Skv=Skv, H=H, Hkv=Hkv, D=D, dtype=ram.RAM_BF16 if dt == "bf16" else ram.RAM_F32,
                 scale=1.0 / math.sqrt(D), softcap=cap or 0.0, causal=causal)
    return dt, d, q, k, v, sinks, src, (qp, kp, qs, ks, causal, cap)


@pytest.mark.parametrize("name", sorted(CHUNK_CASES))
def test_chunk_write(name):
    dt, d, q, k, v, sinks, src, (qp, kp, qs, ks, causal, cap) = _make_chunk_inputs(name)
    say(f"attn_fwd_chunk WRITE {name}")
    out = torch.full((d.B, d.Sq, d.H, d.D), float("nan"), device=DEV)
    lse = torch.full((d.B, d.H, d.Sq), float("nan"), device=DEV)
    _run_chunk(d, q.to(DEV), k.to(DEV), v.to(DEV), src, None if sinks is None else sinks.to(DEV), 0, out, lse)
    torch.cuda.synchronize()
    ro, rl = _chunk_ref(q, k, v, d.scale, qp, kp, qs, ks, causal, cap, sinks)
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, dt, name)


@pytest.mark.parametrize("name", ["bf16_d128_causal_gqa", "bf16_d128_docs_cap_sinks", "f32_d128_segs_cap_sinks",
                                  "bf16_d128_empty_rows", "f32_d64_ragged_gqa"])
def test_chunk_merge_three_chunks(name):
    """WRITE on the first chunk (with sinks), MERGE on the next two == attention over all keys."""
    dt, d, q, k, v, sinks, src, (qp, kp, qs, ks, causal, cap) = _make_chunk_inputs(name)
    say(f"attn_fwd_chunk WRITE+MERGE {name}")
    Skv = d.Skv
    cuts = [0, Skv // 3, (2 * Skv) // 3, Skv]
    out = torch.full((d.B, d.Sq, d.H, d.D), float("nan"), device=DEV)
    lse = torch.full((d.B, d.H, d.Sq), float("nan"), device=DEV)
    kd, vd = k.to(DEV), v.to(DEV)
    for t, (a, e) in enumerate(zip(cuts[:-1], cuts[1:])):
        dc = ram.Desc(**{**d.__dict__, "Skv": e - a, "kv_stride_b": Skv * d.Hkv * d.D})
        sc = ram.MaskSrc(q_pos=src.q_pos, q_pos_base=src.q_pos_base, q_seg=src.q_seg,
                         kv_pos=None if src.kv_pos is None else src.kv_pos[:, a:].contiguous(),
                         kv_pos_base=a,
                         kv_seg=None if src.kv_seg is None else src.kv_seg[:, a:].contiguous(),
                         kv_meta_stride_b=Skv - a)
        # chunk views of k / v: offset base pointer, batch stride of the whole KV
        kc = kd.view(-1)[a * d.Hkv * d.D:]
        vc = vd.view(-1)[a * d.Hkv * d.D:]
        _run_chunk(dc, q.to(DEV), kc, vc, sc, (sinks.to(DEV) if (sinks is not None and t == 0) else None),
                   0 if t == 0 else 1, out, lse)
    torch.cuda.synchronize()
    ro, rl = _chunk_ref(q, k, v, d.scale, qp, kp, qs, ks, causal, cap, sinks)
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, dt, name + " (3 chunks)")


def test_lse_merge_standalone():
    rng = np.random.default_rng(7)
    B, Sq, H, D = 2, 300, 3, 128
    o1 = rng.standard_normal((B, Sq, H, D)).astype(np.float32)
    o2 = rng.standard_normal((B, Sq, H, D)).astype(np.float32)
    l1 = (rng.standard_normal((B, H, Sq)) * 4).astype(np.float32)
    l2 = (rng.standard_normal((B, H, Sq)) * 4).astype(np.float32)
    l1[:, :, :40] = -np.inf                           # running state empty
    l2[:, :, 20:60] = -np.inf                         # block empty (both empty on 20..39)
    o1[np.transpose(l1 == -np.inf, (0, 2, 1))] = 0.0
    o2[np.transpose(l2 == -np.inf, (0, 2, 1))] = 0.0
    l2[:, :, 100:110] = l1[:, :, 100:110]             # equal lse
    ro, rl = oracle.merge(o1, l1, o2, l2)
    ta, tl = torch.from_numpy(o1).to(DEV), torch.from_numpy(l1).to(DEV)
    ram.lse_merge(ta, tl, torch.from_numpy(o2).to(DEV), torch.from_numpy(l2).to(DEV))
    torch.cuda.synchronize()
    go, gl = ta.cpu().numpy().astype(np.float64), tl.cpu().numpy().astype(np.float64)
    assert np.array_equal(gl == -np.inf, rl == -np.inf)
    fin = np.isfinite(rl)
    assert np.max(np.abs(gl[fin] - rl[fin])) <= 2e-6
    assert np.max(np.abs(go - ro)) <= 2e-6
    # a (., -inf) block leaves the running state bit-identical
    assert np.array_equal(go[:, 40:60], o1[:, 40:60])


# ------------------------------------------------------------------------------ ring, small
SMALL_RING = {
    "ring_shard3of4": lambda: wl.c2_ring_shard(Sq=256, H=2, seed=11),
    "ring_shard0of4": lambda: wl.make("s0", B=1, H=2, Hkv=2, Sq=256, chunk=256, n_chunks=4, D=128,
                                      q_shard=0, seed=12),
    "ring_shard1of3_ragged": lambda: wl.make("s1", B=2, H=2, Hkv=1, Sq=200, chunk=200, n_chunks=3, D=128,
                                             q_shard=1, seed=13),
    "docs_small": lambda: wl.c3_packed_docs(S=1024, B=2, H=4, len_lo=32, len_hi=256, seed=14),
    "gqa_cap_sinks_small": lambda: wl.c4_gqa_cap_sinks(S=1024, H=8, Hkv=2, seed=15),
    "mqa_cap_sinks_small": lambda: wl.c4_gqa_cap_sinks(S=1024, H=8, Hkv=1, seed=16),
    "long_small": lambda: wl.c5_long_causal(S=2048, H=4, Hkv=1, seed=17),
    "f32_ring_d64": lambda: wl.make("f32r", B=1, H=2, Hkv=2, Sq=256, chunk=128, n_chunks=2, D=64,
                                    dtype="f32", seed=18, with_sinks=True, softcap=2.0),
    "ragged_chunks_noncausal": lambda: wl.make("nc", B=1, H=2, Hkv=2, Sq=100, chunk=70, n_chunks=3, D=128,
                                               causal=False, seed=19, with_sinks=True),
    # Sq * H / Hkv = 32768 without a cap: V is repacked for row reads; 256 rows of q tiles, so the
    # visits are split over two workgroups; chunks of 1000 keys end inside a 32-key tile
    "packed_v_mqa_split_ragged": lambda: wl.make("pv", B=1, H=8, Hkv=1, Sq=4096, chunk=1000, n_chunks=3, D=128,
                                                 q_shard=1, seed=20),
}


@pytest.mark.parametrize("name", sorted(SMALL_RING))
def test_ring_small(name):
    w = SMALL_RING[name]()
    say(f"ring_attn_fwd_1gpu {name}: B={w.B} H={w.H}/{w.Hkv} Sq={w.Sq} chunks={w.n_chunks}x{w.chunk}")
    out, lse = run_ring(w)
    ro, rl = oracle_ref(w)
    compare(out.numpy(), lse.numpy(), ro, rl, w.dtype, name)


# Rings with enough rows of q tiles for one workgroup per row (no split of the visits).
UNSPLIT_RING = {
    "shard1of4_h64": lambda: wl.make("u1", B=1, H=64, Hkv=8, Sq=1024, chunk=512, n_chunks=4, D=128, q_shard=1,
                                     seed=31),
    "docs_h64": lambda: wl.make("u2", B=2, H=64, Hkv=16, Sq=2048, chunk=512, n_chunks=4, D=128,
                                docs=(64, 700, 0.05), seed=32),
    "cap_sinks_h64": lambda: wl.make("u3", B=1, H=64, Hkv=4, Sq=1024, chunk=384, n_chunks=3, D=128, softcap=30.0,
                                     with_sinks=True, seed=33),
    # Sq * H / Hkv >= 32768 without a cap: the ring reads V repacked (the chunk calls read it as
    # given), so bit-identity checks the repacked operands element for element; ragged chunks
    "packed_v_shard2of4_h64": lambda: wl.make("u4", B=1, H=64, Hkv=2, Sq=1024, chunk=500, n_chunks=4, D=128,
                                              q_shard=2, seed=34),
    "packed_v_docs_h64": lambda: wl.make("u5", B=2, H=64, Hkv=4, Sq=2080, chunk=520, n_chunks=4, D=128,
                                         docs=(64, 700, 0.05), seed=35),
}


@pytest.mark.parametrize("name", sorted(UNSPLIT_RING))
def test_ring_one_launch_equals_chunk_launches(name):
    """The one-launch ring runs every chunk visit as a chunk call does (same tiles, same merge):
    with one workgroup per row its results are bit-identical to attn_fwd_chunk calls in ring
    order (the last merge's float32 output rounded to bf16)."""
    w = UNSPLIT_RING[name]()
    d = ring_desc(w)
    assert not ring_splits(d, w.n_chunks)
    say(f"ring one launch vs chunk calls {name}")
    o1, l1 = run_ring(w)
    sinks = None if w.sinks is None else w.sinks.to(DEV)
    o2, l2 = ring_by_chunks(d, w.n_chunks, w.q_shard, w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), mask_src(w), sinks)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2.to(torch.bfloat16).float().cpu())
    assert torch.equal(l1, l2.cpu())


@pytest.mark.parametrize("name", ["ring_shard3of4", "gqa_cap_sinks_small"])
def test_ring_split_matches_chunk_launches(name):
    """These small rings have fewer rows of q tiles than compute units, so the one-launch ring
    splits each row's visits over two workgroups and merges the halves by their lse: the same
    result as chunk calls in ring order up to the rounding of the merge order (the oracle tests
    check both against the float64 reference)."""
    w = SMALL_RING[name]()
    d = ring_desc(w)
    assert ring_splits(d, w.n_chunks)
    say(f"split ring vs chunk calls {name}")
    o1, l1 = run_ring(w)
    sinks = None if w.sinks is None else w.sinks.to(DEV)
    o2, l2 = ring_by_chunks(d, w.n_chunks, w.q_shard, w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), mask_src(w), sinks)
    torch.cuda.synchronize()
    o2 = o2.to(torch.bfloat16).float().cpu()
    l2 = l2.cpu()
    torch.testing.assert_close(o1, o2, rtol=0, atol=2e-2)
    fin = torch.isfinite(l2)
    assert torch.equal(fin, torch.isfinite(l1))
    torch.testing.assert_close(l1[fin], l2[fin], rtol=0, atol=1e-4)


# ------------------------------------------------------------------------------ full sizes
def test_c1_full():
    w = wl.c1_causal_f32()
    say(f"C1 {w.name}")
    out, lse = run_ring(w)
    ro, rl = oracle_ref(w)
    compare(out.numpy(), lse.numpy(), ro, rl, "f32", w.name)


_C2_REF = {}


def test_c2_full_all_rows():
    w = wl.c2_ring_shard()
    say(f"C2 {w.name}")
    out, lse = run_ring(w)
    if "ref" not in _C2_REF:
        _C2_REF["ref"] = oracle_ref(w)
    ro, rl = _C2_REF["ref"]
    compare(out.numpy(), lse.numpy(), ro, rl, "bf16", w.name)


def test_c3_full_sampled():
    w = wl.c3_packed_docs()
    rows = wl.sampled_rows(w.Sq, 1024, n=384, seed=1003)
    rows = np.unique(np.concatenate([rows, np.arange(w.Sq - 420, w.Sq - 400)]))  # around the padding edge
    say(f"C3 {w.name}: {len(rows)} sampled rows")
    out, lse = run_ring(w)
    ro, rl = oracle_ref(w, rows=rows)
    compare(out.numpy(), lse.numpy(), ro, rl, "bf16", w.name, rows=rows)
    assert np.all(lse.numpy()[:, :, -410:] == -np.inf) and np.all(out.numpy()[:, -410:] == 0)


@pytest.mark.parametrize("Hkv", [8, 1], ids=["gqa8", "mqa"])
def test_c4_full_sampled(Hkv):
    w = wl.c4_gqa_cap_sinks(Hkv=Hkv)
    rows = wl.sampled_rows(w.Sq, w.chunk, n=256, seed=1004)
    say(f"C4 {w.name}: {len(rows)} sampled rows")
    out, lse = run_ring(w)
    ro, rl = oracle_ref(w, rows=rows)
    compare(out.numpy(), lse.numpy(), ro, rl, "bf16", w.name, rows=rows)


def test_c4_error_split():
    """Where C4's output error comes from (GQA with soft cap and sinks, full size, sampled rows):
    the kernel's float32 result (the same ring as attn_fwd_chunk calls, which leave the running
    output in float32) against the oracle, the bf16 rounding of the oracle's own output, and the
    bf16 result against the oracle. The kernel's arithmetic error is bounded by its bf16
    probabilities: each weight p is rounded with relative error <= 2^-9, so the normalised output,
    a convex combination of v rows, moves by at most 2^-9 * max|v| (plus float32 sums)."""
    w = wl.c4_gqa_cap_sinks()
    rows = wl.sampled_rows(w.Sq, w.chunk, n=256, seed=1004)
    d = ring_desc(w)
    src = mask_src(w, DEV)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    sinks = w.sinks.to(DEV)
    o32, l32 = ring_by_chunks(d, w.n_chunks, w.q_shard, q, k, v, src, sinks)
    out, lse = run_ring(w)
    torch.cuda.synchronize()
    ro, rl = oracle_ref(w, rows=rows)
    o32 = o32.cpu().numpy().astype(np.float64)[:, rows]
    o16 = out.numpy().astype(np.float64)[:, rows]
    r16 = torch.from_numpy(ro).to(torch.bfloat16).double().numpy()
    e_kernel = float(np.max(np.abs(o32 - ro)))
    e_round = float(np.max(np.abs(r16 - ro)))
    e_total = float(np.max(np.abs(o16 - ro)))
    e_vs_rounded = float(np.max(np.abs(o16 - r16)))
    bound = 2.0 ** -9 * float(w.v.abs().max()) + 1e-4
    say(f"C4 error split: kernel (float32) {e_kernel:.3e} (bound {bound:.3e}), bf16 rounding of the oracle "
        f"{e_round:.3e}, bf16 result {e_total:.3e} (vs the rounded oracle {e_vs_rounded:.3e})")
    assert e_kernel <= bound
    assert e_total <= OUT_TOL["bf16"]


def test_c5_full_sampled():
    w = wl.c5_long_causal()
    rows = wl.sampled_rows(w.Sq, w.chunk, n=256, seed=1005)
    say(f"C5 {w.name}: {len(rows)} sampled rows")
    out, lse = run_ring(w)
    ro, rl = oracle_ref(w, rows=rows)
    compare(out.numpy(), lse.numpy(), ro, rl, "bf16", w.name, rows=rows)


@pytest.mark.parametrize("dtype,D", [(ram.RAM_BF16, 128), (ram.RAM_F32, 64), (ram.RAM_BF16, 64)])
def test_empty_kv_null_mask_arrays(dtype, D):
    """A chunk of no keys with null tile_class and col_idx (allowed when Skv = 0): every row is
    empty, (0, -inf), and the backward writes dq = 0; no kernel reads the null arrays."""
    import ctypes
    from ring_attention_merge_amd import _lib
    say(f"empty KV, null mask arrays: dtype {dtype} D {D}")
    lib = ram.load()
    B, Sq, H = 2, 300, 2
    tq = torch.bfloat16 if dtype == ram.RAM_BF16 else torch.float32
    bq, bk = ram.kernel_tile(dtype, D)
    d = ram.Desc(B=B, Sq=Sq, Skv=0, H=H, Hkv=H, D=D, dtype=dtype, scale=0.1, causal=False, block_q=bq, block_kv=bk)
    q = torch.randn(B, Sq, H, D, device=DEV).to(tq)
    kv = torch.zeros(16, dtype=tq, device=DEV)
    out = torch.full((B, Sq, H, D), float("nan"), device=DEV)
    lse = torch.full((B, H, Sq), float("nan"), device=DEV)
    row_cnt = torch.zeros(B * (-(-Sq // bq)), dtype=torch.int32, device=DEV)
    bm = _lib.c_block_mask(0, row_cnt.data_ptr(), 0, 0, 0, 0)
    cs = _lib.c_mask_src(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0)
    cd = d.c()
    st = lib.attn_fwd_chunk(ctypes.byref(cd), q.data_ptr(), kv.data_ptr(), kv.data_ptr(), ctypes.byref(cs),
                            ctypes.byref(bm), None, ram.RAM_OUT_WRITE, out.data_ptr(), lse.data_ptr(), None)
    assert st == _lib.RAM_OK, lib.ram_last_error().decode()
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == float("-inf"))
    # the backward of the same chunk: dq of an empty chunk is zero
    bbq, bbk = ram.bwd_kernel_tile(dtype, D)
    db = ram.Desc(**{**d.__dict__, "block_q": bbq, "block_kv": bbk})
    cdb = db.c()
    rcb = torch.zeros(B * (-(-Sq // bbq)), dtype=torch.int32, device=DEV)
    bmb = _lib.c_block_mask(0, rcb.data_ptr(), 0, 0, 0, 0)
    dout = torch.randn(B, Sq, H, D, device=DEV).to(tq)
    delta = torch.zeros(2, B, H, Sq, device=DEV)
    dq = torch.full((B, Sq, H, D), float("nan"), device=DEV)
    st = lib.attn_bwd_chunk(ctypes.byref(cdb), q.data_ptr(), kv.data_ptr(), kv.data_ptr(), dout.data_ptr(),
                            lse.data_ptr(), delta.data_ptr(), ctypes.byref(cs), ctypes.byref(bmb), ram.RAM_OUT_WRITE,
                            dq.data_ptr(), kv.data_ptr(), kv.data_ptr(), None)
    assert st == _lib.RAM_OK, lib.ram_last_error().decode()
    torch.cuda.synchronize()
    assert torch.all(dq == 0)


# ------------------------------------------------------------------------------ invariants
def test_chunked_equals_unchunked_and_order():
    """4 chunks in ring order == 1 chunk of all keys == 4 chunks in natural order (GPU vs GPU)."""
    w = wl.c2_ring_shard(Sq=512, H=4, seed=21)
    o4, l4 = run_ring(w)
    d = ram.Desc(B=1, Sq=512, Skv=2048, H=4, Hkv=4, D=128, scale=w.scale, causal=True)
    outs = []
    for n, shard, base in ((1, -1, 3 * 512), (4, -1, 3 * 512)):
        dd = ram.Desc(**{**d.__dict__, "Skv": 2048 // n})
        out = torch.empty(1, 512, 4, 128, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(1, 4, 512, device=DEV)
        ws = torch.empty(ram.ring_attn_workspace_bytes(dd, n), dtype=torch.uint8, device=DEV)
        ram.ring_attn_fwd_1gpu(dd, n, shard, w.q.to(DEV), w.k.to(DEV), w.v.to(DEV),
                               ram.MaskSrc(q_pos_base=base), None, out, lse, ws)
        torch.cuda.synchronize()
        outs.append((out.float().cpu().numpy(), lse.cpu().numpy()))
    for o, l in outs:
        assert np.max(np.abs(o - o4.numpy())) <= 1e-2
        assert np.max(np.abs(l - l4.numpy())) <= 1e-4


def test_gqa_equals_repeated_kv_bitwise():
    w = wl.c4_gqa_cap_sinks(S=1024, H=8, Hkv=2, seed=22)
    o1, l1 = run_ring(w)
    w.k = w.k.repeat_interleave(4, dim=2).contiguous()
    w.v = w.v.repeat_interleave(4, dim=2).contiguous()
    w.Hkv = 8
    o2, l2 = run_ring(w)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_deterministic():
    w = wl.c3_packed_docs(S=2048, B=2, H=4, len_lo=64, len_hi=512, seed=23)
    o1, l1 = run_ring(w)
    o2, l2 = run_ring(w)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_all_pad_batch_and_empty_kv():
    w = wl.c3_packed_docs(S=512, B=2, H=2, len_lo=32, len_hi=128, seed=24)
    w.q_seg = w.q_seg.copy()
    w.q_seg[1] = -1                                   # batch 1 entirely padding
    w.kv_seg = w.q_seg
    out, lse = run_ring(w)
    assert np.all(lse.numpy()[1] == -np.inf) and np.all(out.numpy()[1] == 0)
    ro, rl = oracle_ref(w)
    compare(out.numpy(), lse.numpy(), ro, rl, "bf16", "all-pad batch")
    # Skv = 0: every row empty; with sinks the row is (0, sink)
    for with_sinks in (False, True):
        d = ram.Desc(B=1, Sq=130, Skv=0, H=2, Hkv=1, D=128, scale=0.1)
        out = torch.full((1, 130, 2, 128), float("nan"), device=DEV)
        lse = torch.full((1, 2, 130), float("nan"), device=DEV)
        sinks = torch.tensor([0.5, -2.0], device=DEV) if with_sinks else None
        q = torch.randn(1, 130, 2, 128, device=DEV).to(torch.bfloat16)
        _run_chunk(d, q, None, None, ram.MaskSrc(), sinks, 0, out, lse)
        torch.cuda.synchronize()
        assert torch.all(out == 0)
        if with_sinks:
            exp = torch.tensor([0.5, -2.0])[None, :, None].expand(1, 2, 130)
            assert torch.allclose(lse.cpu(), exp, rtol=0, atol=1e-6)
        else:
            assert torch.all(lse.cpu() == -math.inf)
