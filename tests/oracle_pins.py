"""Pins for the float64 oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` takes an oracle module ``ora`` (with ``attention``, ``allowed``,
``merge``, ``chunked``, ``block_mask``, ``partial_bits`` and the tile-class
constants) and raises
AssertionError when the oracle disagrees with:
  * the constants the pages print (tests/golden/*.json),
  * closed forms (zero queries, single allowed key, constant values, merge as
    logaddexp plus a weighted mean, the soft cap on two keys),
  * library routines (torch scaled_dot_product_attention and logsumexp in
    float64, numpy reshapes for the tile classes),
  * brute force with math.fsum on tiny inputs,
  * invariants (chunked + merge equals the whole KV in any split and order,
    GQA equals repeated KV heads, packed documents equal separate documents,
    ring offsets equal one offset causal mask, a sink counts once, a
    lower-triangular dense mask equals the causal test, a block-diagonal one
    equals segment IDs, a reused local mask equals the tiled global one),
  * numpy's little-endian bit unpacking for the partial-tile bits.
``tests/test_oracle_pins.py`` runs them on the real oracle;
``tests/test_oracle_mutants.py`` runs them on broken copies and expects failures.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from ring_attention_merge_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FLT_MAX = float(np.finfo(np.float32).max)
PAD = -1


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb), f"{what}: finite pattern differs"
    assert np.array_equal(a[~fa], b[~fb]), f"{what}: non-finite values differ"
    if fa.any():
        err = np.max(np.abs(a[fa] - b[fb]))
        assert err <= tol, f"{what}: max err {err:.3e} > {tol:.1e}"


def _rand_problem(rng, B, Sq, Skv, H, Hkv, D, *, segs=False, shuffle_pos=False, pad=False):
    q = rng.standard_normal((B, Sq, H, D))
    k = rng.standard_normal((B, Skv, Hkv, D))
    v = rng.standard_normal((B, Skv, Hkv, D))
    if shuffle_pos:
        qp = rng.integers(0, max(Sq, Skv), size=(B, Sq))
        kp = rng.integers(0, max(Sq, Skv), size=(B, Skv))
    else:
        qp = np.broadcast_to(np.arange(Sq) + (Skv - Sq if Skv > Sq else 0), (B, Sq)).copy()
        kp = np.broadcast_to(np.arange(Skv), (B, Skv)).copy()
    qs = ks = None
    if segs:
        qs = rng.integers(0, 3, size=(B, Sq))
        ks = rng.integers(0, 3, size=(B, Skv))
        if pad:
            qs[rng.random((B, Sq)) < 0.2] = PAD
            ks[rng.random((B, Skv)) < 0.2] = PAD
    return q, k, v, qp, kp, qs, ks


def _mask_indep(qp, kp, qs, ks, causal):
    """The element mask written as set membership (independent of ``ora.allowed``)."""
    Sq, Skv = len(qp), len(kp)
    m = np.zeros((Sq, Skv), bool)
    for i in range(Sq):
        for j in range(Skv):
            ok = (not causal) or not (kp[j] > qp[i])
            if qs is not None:
                ok = ok and qs[i] != PAD and qs[i] == ks[j]
            m[i, j] = ok
    return m


# ---------------------------------------------------------------------------- constants
def pin_mask_value_constant(ora):
    g = _golden("mask_value.json")["value"]
    assert ora.DEFAULT_MASK_VALUE == g, "mask value differs from the printed constant"
    assert abs(g - (-0.7 * FLT_MAX)) <= 1e-15 * abs(g), "printed mask value is not -0.7*FLT_MAX"
    assert np.isfinite(np.float32(g))


def pin_finite_mask_equivalence(ora):
    """Exact exclusion equals the pages' finite mask value (fp32) on rows with >=1 key."""
    rng = np.random.default_rng(11)
    q, k, v, qp, kp, qs, ks = _rand_problem(rng, 1, 24, 24, 2, 2, 8, segs=True, pad=True)
    scale = 0.3
    out, lse = ora.attention(q, k, v, scale=scale, q_pos=qp, kv_pos=kp, q_seg=qs, kv_seg=ks)
    mv = _golden("mask_value.json")["value"]
    m = _mask_indep(qp[0], kp[0], qs[0], ks[0], True)
    for h in range(2):
        s = scale * torch.from_numpy(q[0, :, h]).float() @ torch.from_numpy(k[0, :, h]).float().T
        s = torch.where(torch.from_numpy(m), s, torch.tensor(mv, dtype=torch.float32))
        p = torch.softmax(s, dim=-1)
        o = (p @ torch.from_numpy(v[0, :, h]).float()).double().numpy()
        rows = m.any(axis=1)
        assert rows.any() and (~rows).any()
        _close(out[0, rows, h], o[rows], 2e-6, "finite mask value")


# ---------------------------------------------------------------------------- brute force
def _brute(q, k, v, scale, qp, kp, qs, ks, causal, cap, sinks):
    B, Sq, H, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    out = np.zeros((B, Sq, H, D))
    lse = np.full((B, H, Sq), -math.inf)
    for b in range(B):
        for h in range(H):
            g = (h * Hkv) // H
            for i in range(Sq):
                ws, js = [], []
                for j in range(Skv):
                    if causal and kp[b, j] > qp[b, i]:
                        continue
                    if qs is not None and (qs[b, i] == PAD or qs[b, i] != ks[b, j]):
                        continue
                    s = scale * math.fsum(float(q[b, i, h, d]) * float(k[b, j, g, d]) for d in range(D))
                    if cap is not None:
                        s = cap * math.tanh(s / cap)
                    ws.append(math.exp(s))
                    js.append(j)
                terms = list(ws) + ([math.exp(float(sinks[h]))] if sinks is not None else [])
                if not terms:
                    continue
                Z = math.fsum(terms)
                lse[b, h, i] = math.log(Z)
                for d in range(D):
                    out[b, i, h, d] = math.fsum(w * float(v[b, j, g, d]) for w, j in zip(ws, js)) / Z
    return out, lse


def pin_bruteforce(ora):
    rng = np.random.default_rng(12)
    for trial in range(24):
        B = int(rng.integers(1, 3))
        Hkv = int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2, 3]))
        Sq, Skv, D = (int(x) for x in rng.integers(1, 10, size=3))
        segs = bool(rng.integers(0, 2))
        q, k, v, qp, kp, qs, ks = _rand_problem(rng, B, Sq, Skv, H, Hkv, D, segs=segs,
                                                shuffle_pos=bool(rng.integers(0, 2)), pad=segs)
        causal = bool(rng.integers(0, 2))
        cap = float(rng.choice([0.7, 3.0])) if rng.integers(0, 2) else None
        sinks = rng.standard_normal(H) if rng.integers(0, 2) else None
        scale = float(rng.uniform(0.2, 1.0))
        o1, l1 = ora.attention(q, k, v, scale=scale, q_pos=qp, kv_pos=kp, q_seg=qs, kv_seg=ks,
                               causal=causal, softcap=cap, sinks=sinks)
        o2, l2 = _brute(q, k, v, scale, qp, kp, qs, ks, causal, cap, sinks)
        _close(o1, o2, 1e-12, f"brute out trial {trial}")
        _close(l1, l2, 1e-12, f"brute lse trial {trial}")


# ---------------------------------------------------------------------------- library routines
def pin_sdpa(ora):
    """No cap, no sinks: out equals torch SDPA (float64, GQA), lse equals torch logsumexp."""
    rng = np.random.default_rng(13)
    B, Sq, Skv, H, Hkv, D = 2, 70, 83, 4, 2, 16
    q, k, v, qp, kp, qs, ks = _rand_problem(rng, B, Sq, Skv, H, Hkv, D, segs=True, pad=True)
    scale = 0.25
    out, lse = ora.attention(q, k, v, scale=scale, q_pos=qp, kv_pos=kp, q_seg=qs, kv_seg=ks)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    mask = torch.from_numpy(np.stack([_mask_indep(qp[b], kp[b], qs[b], ks[b], True)
                                      for b in range(B)]))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                                          enable_gqa=True)
    ref = ref.permute(0, 2, 1, 3).numpy()
    rows = mask[:, 0].any(-1).numpy()                       # [B,Sq]
    assert rows.any() and (~rows).any()
    for b in range(B):
        _close(out[b, rows[b]], ref[b, rows[b]], 1e-12, "sdpa out")
    kr = tk.repeat_interleave(H // Hkv, dim=1)
    s = scale * (tq @ kr.transpose(-1, -2))
    s = s.masked_fill(~mask, -math.inf)
    ref_lse = torch.logsumexp(s, dim=-1).numpy()            # [B,H,Sq]
    _close(lse, ref_lse, 1e-12, "logsumexp lse")


# ---------------------------------------------------------------------------- closed forms
def pin_closed_forms(ora):
    rng = np.random.default_rng(14)
    B, S, H, D = 1, 40, 2, 8
    # zero queries, sequential causal: row i averages keys 0..i and lse = ln(i+1)
    q = np.zeros((B, S, H, D))
    k = rng.standard_normal((B, S, H, D))
    v = rng.standard_normal((B, S, H, D))
    pos = np.arange(S)[None]
    out, lse = ora.attention(q, k, v, scale=0.7, q_pos=pos, kv_pos=pos, softcap=5.0)
    cm = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    _close(out, cm, 1e-12, "zero-q mean")
    _close(lse, np.broadcast_to(np.log(np.arange(1, S + 1)), (B, H, S)), 1e-12, "zero-q lse")
    # one allowed key per row: out is that value row, lse that logit
    q = rng.standard_normal((B, S, H, D))
    seg = np.arange(S)[None]
    kperm = rng.permutation(S)
    out, lse = ora.attention(q, k, v, scale=0.3, q_pos=pos, kv_pos=pos, q_seg=seg,
                             kv_seg=seg[:, kperm], causal=False)
    inv = np.argsort(kperm)                                  # key holding segment i
    for h in range(H):
        for i in range(S):
            j = inv[i]
            s = 0.3 * math.fsum(q[0, i, h, d] * k[0, j, h, d] for d in range(D))
            assert abs(lse[0, h, i] - s) <= 1e-12
            assert np.array_equal(out[0, i, h], v[0, j, h])
    # constant values give the constant back; rows with nothing allowed give (0, -inf)
    vc = np.full((B, S, H, D), 0.625)
    qp = pos.copy()
    qp[0, :5] = -1                                           # before every key: nothing allowed
    out, lse = ora.attention(q, k, vc, scale=0.3, q_pos=qp, kv_pos=pos)
    _close(out[0, 5:], vc[0, 5:], 1e-12, "constant v")
    assert np.all(out[0, :5] == 0) and np.all(lse[0, :, :5] == -np.inf)
    sinks = np.array([0.25, -1.5])
    out, lse = ora.attention(q, k, vc, scale=0.3, q_pos=qp, kv_pos=pos, sinks=sinks)
    assert np.all(out[0, :5] == 0) and np.array_equal(lse[0, :, :5], np.repeat(sinks[:, None], 5, 1))


def pin_softcap(ora):
    """Two allowed keys: lse = ln(e^c(s1) + e^c(s2)), c(s) = cap*tanh(s/cap); large cap -> uncapped."""
    cap = 2.0
    q = np.zeros((1, 1, 1, 2)); q[0, 0, 0] = [1.5, -0.5]
    k = np.zeros((1, 2, 1, 2)); k[0, 0, 0] = [2.0, 1.0]; k[0, 1, 0] = [-1.0, 3.0]
    v = np.zeros((1, 2, 1, 1)); v[0, 0, 0, 0] = 1.0; v[0, 1, 0, 0] = -2.0
    s1 = 0.5 * (1.5 * 2.0 - 0.5 * 1.0)
    s2 = 0.5 * (1.5 * -1.0 - 0.5 * 3.0)
    c1, c2 = cap * math.tanh(s1 / cap), cap * math.tanh(s2 / cap)
    out, lse = ora.attention(q, k, v, scale=0.5, q_pos=np.array([[5]]), kv_pos=np.array([[0, 1]]),
                             softcap=cap)
    ref_lse = math.log(math.exp(c1) + math.exp(c2))
    assert abs(lse[0, 0, 0] - ref_lse) <= 1e-13, (lse, ref_lse)
    w1 = math.exp(c1 - ref_lse)
    assert abs(out[0, 0, 0, 0] - (w1 * 1.0 + (1 - w1) * -2.0)) <= 1e-13
    rng = np.random.default_rng(15)
    q, k, v, qp, kp, _, _ = _rand_problem(rng, 1, 16, 16, 2, 2, 4)
    o1, l1 = ora.attention(q, k, v, scale=0.5, q_pos=qp, kv_pos=kp, softcap=1e7)
    o2, l2 = ora.attention(q, k, v, scale=0.5, q_pos=qp, kv_pos=kp)
    _close(o1, o2, 1e-9, "large cap"); _close(l1, l2, 1e-9, "large cap lse")
    o3, _ = ora.attention(q, k, v, scale=0.5, q_pos=qp, kv_pos=kp, softcap=1.0)
    assert np.max(np.abs(o3 - o2)) > 1e-3, "cap has no effect"


# ---------------------------------------------------------------------------- merge
def pin_merge(ora):
    g = _golden("merge_example.json")
    o = np.zeros((1, 1, 1, 1)); bo = np.ones((1, 1, 1, 1))
    _, nl = ora.merge(o, np.full((1, 1, 1), g["lse"]), bo, np.full((1, 1, 1), g["block_lse"]))
    assert abs(nl[0, 0, 0] - g["merged_lse"]) <= g["tol"], nl
    rng = np.random.default_rng(16)
    B, S, H, D = 2, 9, 3, 5
    out = rng.standard_normal((B, S, H, D)); bo = rng.standard_normal((B, S, H, D))
    lse = rng.standard_normal((B, H, S)) * 3; bl = rng.standard_normal((B, H, S)) * 3
    no, nl = ora.merge(out, lse, bo, bl)
    ref_l = np.logaddexp(lse, bl)
    wa = np.exp(lse - ref_l).transpose(0, 2, 1)[..., None]
    wb = np.exp(bl - ref_l).transpose(0, 2, 1)[..., None]
    _close(nl, ref_l, 1e-12, "merge lse = logaddexp")
    _close(no, wa * out + wb * bo, 1e-12, "merge out = weighted mean")
    # commutative up to rounding
    no2, nl2 = ora.merge(bo, bl, out, lse)
    _close(no2, no, 1e-12, "merge commutes"); _close(nl2, nl, 1e-12, "merge commutes lse")
    # special cases: a (., -inf) block is the identity; -inf running state adopts; both -inf
    ninf = np.full((B, H, S), -np.inf)
    o1, l1 = ora.merge(out, lse, np.zeros_like(bo), ninf)
    assert np.array_equal(o1, out) and np.array_equal(l1, lse)
    o2, l2 = ora.merge(np.zeros_like(out), ninf, bo, bl)
    assert np.array_equal(o2, bo) and np.array_equal(l2, bl)
    o3, l3 = ora.merge(np.zeros_like(out), ninf, np.zeros_like(bo), ninf)
    assert np.all(o3 == 0) and np.all(l3 == -np.inf)
    o4, l4 = ora.merge(out, lse, bo, lse)
    _close(o4, 0.5 * (out + bo), 1e-12, "equal lse average")
    _close(l4, lse + math.log(2), 1e-12, "equal lse + ln2")


# ---------------------------------------------------------------------------- invariants
def pin_chunked_equals_full(ora):
    rng = np.random.default_rng(17)
    for trial in range(6):
        B, Sq, H, Hkv, D = 1 + trial % 2, 20 + trial, 4, 2, 8
        Skv = int(rng.integers(30, 60))
        q, k, v, qp, kp, qs, ks = _rand_problem(rng, B, Sq, Skv, H, Hkv, D, segs=trial >= 3,
                                                shuffle_pos=trial % 3 == 2, pad=trial >= 3)
        cap = 4.0 if trial % 2 else None
        sinks = rng.standard_normal(H) if trial % 3 else None
        cuts = np.sort(rng.choice(np.arange(1, Skv), size=3, replace=False))
        edges = [0, *cuts.tolist(), Skv]
        bounds = [(edges[i], edges[i + 1]) for i in range(4)]
        ref_o, ref_l = ora.attention(q, k, v, scale=0.4, q_pos=qp, kv_pos=kp, q_seg=qs, kv_seg=ks,
                                     softcap=cap, sinks=sinks)
        for order in ([0, 1, 2, 3], [3, 2, 1, 0], list(rng.permutation(4))):
            o, l = ora.chunked(q, k, v, scale=0.4, q_pos=qp, kv_pos=kp, bounds=bounds, order=order,
                               q_seg=qs, kv_seg=ks, softcap=cap, sinks=sinks)
            _close(o, ref_o, 1e-12, f"chunked out {order}")
            _close(l, ref_l, 1e-12, f"chunked lse {order}")


def pin_sink_once(ora):
    """A sink is a virtual chunk (out 0, lse sink); it counts once, not per chunk."""
    rng = np.random.default_rng(18)
    B, S, H, D = 1, 32, 2, 8
    q, k, v, qp, kp, _, _ = _rand_problem(rng, B, S, S, H, H, D)
    sinks = rng.standard_normal(H) * 2
    o0, l0 = ora.attention(q, k, v, scale=0.35, q_pos=qp, kv_pos=kp)
    o1, l1 = ora.attention(q, k, v, scale=0.35, q_pos=qp, kv_pos=kp, sinks=sinks)
    sk = sinks[None, :, None]
    _close(l1, np.logaddexp(l0, sk), 1e-12, "sink lse = logaddexp(lse, sink)")
    w = (1.0 / (1.0 + np.exp(sk - l0))).transpose(0, 2, 1)[..., None]
    _close(o1, o0 * w, 1e-12, "sink out = out * sigmoid(lse - sink)")
    bounds = [(0, 8), (8, 16), (16, 24), (24, 32)]
    # sink on every chunk: must differ from the single sink
    acc, acc_l = np.zeros_like(o0), np.full_like(l0, -np.inf)
    for a, e in bounds:
        oc, lc = ora.attention(q, k[:, a:e], v[:, a:e], scale=0.35, q_pos=qp, kv_pos=kp[:, a:e],
                               sinks=sinks)
        acc, acc_l = ora.merge(acc, acc_l, oc, lc)
    assert np.max(np.abs(acc_l - l1)) > 1e-2, "sink counted per chunk is indistinguishable"
    # the pages' later-step sentinel gives the same result as no sink where a key is allowed
    sent = _golden("sink_sentinel.json")["value"]
    oc, lc = ora.attention(q, k[:, 8:16], v[:, 8:16], scale=0.35, q_pos=qp, kv_pos=kp[:, 8:16],
                           sinks=np.full(H, sent))
    on, ln = ora.attention(q, k[:, 8:16], v[:, 8:16], scale=0.35, q_pos=qp, kv_pos=kp[:, 8:16])
    rows = np.isfinite(ln[0, 0])
    _close(oc[:, rows], on[:, rows], 1e-12, "sentinel out"); _close(lc[..., rows], ln[..., rows], 1e-12, "sentinel lse")


def pin_gqa_repeat(ora):
    rng = np.random.default_rng(19)
    for H, Hkv in ((8, 2), (6, 1), (4, 4)):
        q, k, v, qp, kp, qs, ks = _rand_problem(rng, 1, 18, 22, H, Hkv, 4, segs=True, pad=True)
        o1, l1 = ora.attention(q, k, v, scale=0.5, q_pos=qp, kv_pos=kp, q_seg=qs, kv_seg=ks, softcap=3.0)
        kr, vr = np.repeat(k, H // Hkv, axis=2), np.repeat(v, H // Hkv, axis=2)
        o2, l2 = ora.attention(q, kr, vr, scale=0.5, q_pos=qp, kv_pos=kp, q_seg=qs, kv_seg=ks, softcap=3.0)
        _close(o1, o2, 0.0, f"gqa {H}/{Hkv}"); _close(l1, l2, 0.0, f"gqa lse {H}/{Hkv}")


def pin_packed_docs(ora):
    rng = np.random.default_rng(20)
    S, H, D = 96, 2, 8
    seg, pos, lengths = wl.packed_documents(rng, 1, S, 5, 30, 0.1)
    q = rng.standard_normal((1, S, H, D)); k = rng.standard_normal((1, S, H, D)); v = rng.standard_normal((1, S, H, D))
    out, lse = ora.attention(q, k, v, scale=0.4, q_pos=pos, kv_pos=pos, q_seg=seg, kv_seg=seg)
    t = 0
    for L in lengths[0]:
        p = np.arange(L)[None]
        o, l = ora.attention(q[:, t:t + L], k[:, t:t + L], v[:, t:t + L], scale=0.4, q_pos=p, kv_pos=p)
        _close(out[:, t:t + L], o, 1e-12, "document slice"); _close(lse[:, :, t:t + L], l, 1e-12, "doc lse")
        t += L
    assert t < S
    assert np.all(out[:, t:] == 0) and np.all(lse[:, :, t:] == -np.inf), "pad rows"


def pin_ring_offsets(ora):
    """Shard r of N in ring order (r - t) mod N equals one causal mask offset by r*Sq."""
    rng = np.random.default_rng(21)
    N, Sq, H, D = 4, 12, 2, 8
    for r in range(N):
        q = rng.standard_normal((1, Sq, H, D))
        k = rng.standard_normal((1, N * Sq, H, D)); v = rng.standard_normal((1, N * Sq, H, D))
        qp = (r * Sq + np.arange(Sq))[None]
        kp = np.arange(N * Sq)[None]
        bounds = [(c * Sq, (c + 1) * Sq) for c in range(N)]
        order = [(r - t) % N for t in range(N)]
        o, l = ora.chunked(q, k, v, scale=0.3, q_pos=qp, kv_pos=kp, bounds=bounds, order=order)
        mask = torch.ones(Sq, N * Sq, dtype=torch.bool).tril(diagonal=r * Sq)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q).permute(0, 2, 1, 3), torch.from_numpy(k).permute(0, 2, 1, 3),
            torch.from_numpy(v).permute(0, 2, 1, 3), attn_mask=mask, scale=0.3).permute(0, 2, 1, 3)
        _close(o, ref.numpy(), 1e-12, f"ring shard {r}")
        s = 0.3 * torch.from_numpy(q).permute(0, 2, 1, 3) @ torch.from_numpy(k).permute(0, 2, 3, 1)
        ref_l = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
        _close(l, ref_l.numpy(), 1e-12, f"ring shard {r} lse")


# ---------------------------------------------------------------------------- block mask
def _classes_by_reshape(ok, bq, bk):
    Sq, Skv = ok.shape
    nQb, nKb = -(-Sq // bq), -(-Skv // bk)
    anyp = np.zeros((nQb * bq, nKb * bk), bool); anyp[:Sq, :Skv] = ok
    allp = np.ones((nQb * bq, nKb * bk), bool); allp[:Sq, :Skv] = ok
    a = anyp.reshape(nQb, bq, nKb, bk).any(axis=(1, 3))
    f = allp.reshape(nQb, bq, nKb, bk).all(axis=(1, 3))
    return np.where(f, 2, np.where(a, 1, 0)).astype(np.uint8)


def pin_block_mask(ora):
    rng = np.random.default_rng(22)
    # sequential causal: FULL iff min q_pos >= max kv_pos, EMPTY iff max q_pos < min kv_pos
    for trial in range(30):
        Sq, Skv = (int(x) for x in rng.integers(1, 300, size=2))
        bq, bk = int(rng.choice([16, 32, 64, 128])), int(rng.choice([16, 32, 64, 128]))
        qb0, kb0 = int(rng.integers(0, 400)), int(rng.integers(0, 400))
        qp, kp = qb0 + np.arange(Sq), kb0 + np.arange(Skv)
        cls, cnt, col = ora.block_mask(ora.allowed(qp, kp, causal=True), bq, bk)
        nQb, nKb = -(-Sq // bq), -(-Skv // bk)
        exp = np.zeros((nQb, nKb), np.uint8)
        for i in range(nQb):
            qlo, qhi = qb0 + i * bq, qb0 + min(Sq, (i + 1) * bq) - 1
            for j in range(nKb):
                klo, khi = kb0 + j * bk, kb0 + min(Skv, (j + 1) * bk) - 1
                exp[i, j] = ora.TILE_FULL if qlo >= khi else (ora.TILE_EMPTY if qhi < klo else ora.TILE_PARTIAL)
        assert np.array_equal(cls, exp), f"closed-form classes, trial {trial}"
        for i in range(nQb):
            nz = np.nonzero(exp[i])[0]
            assert cnt[i] == len(nz) and np.array_equal(col[i, :len(nz)], nz)
            assert np.all(col[i, len(nz):] == -1)
    # square causal, aligned tiles: n(n+1)/2 non-empty, n of them PARTIAL (the diagonal)
    for n, b in ((16, 128), (24, 64)):
        p = np.arange(n * b)
        cls, cnt, _ = ora.block_mask(ora.allowed(p, p), b, b)
        assert int(cnt.sum()) == n * (n + 1) // 2 and int((cls == ora.TILE_PARTIAL).sum()) == n
    # ring shard 3 of 4 at 128x128 over chunks of 4096 keys: 528 tiles on the diagonal chunk
    qp = 3 * 4096 + np.arange(4096)
    for c, want in ((3, 528), (2, 1024), (0, 1024)):
        cls, cnt, _ = ora.block_mask(ora.allowed(qp, c * 4096 + np.arange(4096)), 128, 128)
        assert int(cnt.sum()) == want, (c, int(cnt.sum()))
    # general positions and segments: equal to the any/all-over-reshape classes
    for trial in range(10):
        Sq, Skv = (int(x) for x in rng.integers(1, 200, size=2))
        qs = rng.integers(-1, 3, size=Sq); ks = rng.integers(-1, 3, size=Skv)
        qs[: Sq // 2] = 1; ks[: Skv // 2] = 1
        qp = rng.integers(0, 150, size=Sq); kp = rng.integers(0, 150, size=Skv)
        ok = _mask_indep(qp, kp, qs, ks, True)
        cls, _, _ = ora.block_mask(ora.allowed(qp, kp, qs, ks, True), 32, 16)
        assert np.array_equal(cls, _classes_by_reshape(ok, 32, 16)), f"segment classes {trial}"


# ---------------------------------------------------------------------------- dense masks
def _brute_dense(q, k, v, scale, dense, causal, qp, kp):
    """Brute force with a dense mask shared by all batch rows (no cap, sinks or segments)."""
    B, Sq, H, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    out = np.zeros((B, Sq, H, D))
    lse = np.full((B, H, Sq), -math.inf)
    for b in range(B):
        for h in range(H):
            g = (h * Hkv) // H
            for i in range(Sq):
                ws, js = [], []
                for j in range(Skv):
                    if not dense[i][j] or (causal and kp[b, j] > qp[b, i]):
                        continue
                    s = scale * math.fsum(float(q[b, i, h, d]) * float(k[b, j, g, d]) for d in range(D))
                    ws.append(math.exp(s))
                    js.append(j)
                if not ws:
                    continue
                Z = math.fsum(ws)
                lse[b, h, i] = math.log(Z)
                for d in range(D):
                    out[b, i, h, d] = math.fsum(w * float(v[b, j, g, d]) for w, j in zip(ws, js)) / Z
    return out, lse


def pin_dense_mask(ora):
    rng = np.random.default_rng(23)
    # brute force on tiny inputs, one mask for both batch rows, Sq != Skv
    for trial in range(12):
        B, Hkv = 2, int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2]))
        Sq, Skv, D = int(rng.integers(1, 9)), int(rng.integers(1, 11)), int(rng.integers(1, 6))
        q, k, v, qp, kp, _, _ = _rand_problem(rng, B, Sq, Skv, H, Hkv, D, shuffle_pos=True)
        dense = (rng.random((Sq, Skv)) < 0.6).astype(np.uint8) * int(rng.choice([1, 3]))
        causal = bool(trial % 2)
        o1, l1 = ora.attention(q, k, v, scale=0.45, q_pos=qp, kv_pos=kp, causal=causal, dense=dense)
        o2, l2 = _brute_dense(q, k, v, 0.45, dense, causal, qp, kp)
        _close(o1, o2, 1e-12, f"dense brute out {trial}"); _close(l1, l2, 1e-12, f"dense brute lse {trial}")
    # a lower-triangular mask (numpy tri, offset by the q shift) equals the causal test
    Sq, Skv, off = 37, 53, 16
    q, k, v, _, _, _, _ = _rand_problem(rng, 1, Sq, Skv, 2, 1, 8)
    qp, kp = (off + np.arange(Sq))[None], np.arange(Skv)[None]
    tri = np.tri(Sq, Skv, k=off, dtype=bool)
    o1, l1 = ora.attention(q, k, v, scale=0.3, q_pos=qp, kv_pos=kp, causal=False, dense=tri)
    o2, l2 = ora.attention(q, k, v, scale=0.3, q_pos=qp, kv_pos=kp, causal=True)
    _close(o1, o2, 0.0, "tri dense = causal"); _close(l1, l2, 0.0, "tri dense = causal lse")
    # a block-diagonal mask (scipy block_diag of documents) equals segment IDs
    import scipy.linalg
    S = 90
    seg, pos, lengths = wl.packed_documents(rng, 1, S, 7, 25, 0.1)
    bd = scipy.linalg.block_diag(*[np.ones((L, L)) for L in lengths[0]])
    dense = np.zeros((S, S)); dense[:bd.shape[0], :bd.shape[1]] = bd
    q, k, v, _, _, _, _ = _rand_problem(rng, 1, S, S, 2, 2, 8)
    o1, l1 = ora.attention(q, k, v, scale=0.3, q_pos=pos, kv_pos=pos, causal=False, dense=dense)
    o2, l2 = ora.attention(q, k, v, scale=0.3, q_pos=pos, kv_pos=pos, q_seg=seg, kv_seg=seg, causal=False)
    _close(o1, o2, 0.0, "block-diagonal = segments"); _close(l1, l2, 0.0, "block-diagonal = segments lse")
    # dense AND causal AND segments: the intersection of the three element masks
    o1, l1 = ora.attention(q, k, v, scale=0.3, q_pos=pos, kv_pos=pos, q_seg=seg, kv_seg=seg,
                           causal=True, dense=np.tri(S, S, k=-2))
    pos2 = np.arange(S)[None]
    both = _mask_indep(pos[0], pos[0], seg[0], seg[0], True) & np.tri(S, S, k=-2, dtype=bool)
    o2, l2 = ora.attention(q, k, v, scale=0.3, q_pos=pos2, kv_pos=pos2, causal=False, dense=both)
    _close(o1, o2, 0.0, "intersection"); _close(l1, l2, 0.0, "intersection lse")
    # a cleared row gives (0, -inf); with a sink, lse = sink
    dense = np.ones((S, S), np.uint8); dense[5] = 0
    sinks = np.array([0.5, -2.0])
    o, l = ora.attention(q, k, v, scale=0.3, q_pos=pos2, kv_pos=pos2, dense=dense)
    assert np.all(o[0, 5] == 0) and np.all(l[0, :, 5] == -np.inf)
    o, l = ora.attention(q, k, v, scale=0.3, q_pos=pos2, kv_pos=pos2, dense=dense, sinks=sinks)
    assert np.all(o[0, 5] == 0) and np.array_equal(l[0, :, 5], sinks)


def pin_dense_chunked(ora):
    rng = np.random.default_rng(24)
    N, C, Sq, H, D = 4, 13, 21, 2, 8
    q, k, v, _, _, _, _ = _rand_problem(rng, 1, Sq, N * C, H, H, D)
    qp, kp = (3 * C + np.arange(Sq))[None], np.arange(N * C)[None]
    bounds = [(c * C, (c + 1) * C) for c in range(N)]
    for causal in (False, True):
        # one mask over the whole KV: each chunk reads its own columns
        dense = rng.random((Sq, N * C)) < 0.5
        ref_o, ref_l = ora.attention(q, k, v, scale=0.3, q_pos=qp, kv_pos=kp, causal=causal, dense=dense)
        for order in ([0, 1, 2, 3], [3, 2, 1, 0], [1, 3, 0, 2]):
            o, l = ora.chunked(q, k, v, scale=0.3, q_pos=qp, kv_pos=kp, bounds=bounds, order=order,
                               causal=causal, dense=dense)
            _close(o, ref_o, 1e-12, f"global dense {order}"); _close(l, ref_l, 1e-12, f"global dense lse {order}")
        # one local mask reused at every step equals that mask tiled along the keys
        local = rng.random((Sq, C)) < 0.5
        ref_o, ref_l = ora.attention(q, k, v, scale=0.3, q_pos=qp, kv_pos=kp, causal=causal,
                                     dense=np.tile(local, (1, N)))
        o, l = ora.chunked(q, k, v, scale=0.3, q_pos=qp, kv_pos=kp, bounds=bounds, order=[3, 2, 1, 0],
                           causal=causal, dense=local, dense_col0=[0] * N)
        _close(o, ref_o, 1e-12, "reused local dense"); _close(l, ref_l, 1e-12, "reused local dense lse")


def pin_partial_bits(ora):
    rng = np.random.default_rng(25)
    for trial in range(16):
        Sq, Skv = (int(x) for x in rng.integers(1, 160, size=2))
        bq, bk = int(rng.choice([16, 32, 48])), int(rng.choice([16, 32, 48, 64, 100]))
        ok = rng.random((Sq, Skv)) < rng.choice([0.05, 0.5, 0.97])
        ok[: Sq // 3, : Skv // 3] = True                                   # some FULL tiles
        ok[Sq // 2:, Skv // 2:] = False                                    # some EMPTY tiles
        bits = ora.partial_bits(ok, bq, bk)
        cls = _classes_by_reshape(ok, bq, bk)
        nQb, nKb = cls.shape
        W = -(-bk // 32)
        assert bits.shape == (nQb, nKb, bq, W) and bits.dtype == np.uint32
        # numpy's little-endian unpacking: bit j of the row is key j of the tile
        unp = np.unpackbits(bits.astype("<u4").view(np.uint8), axis=-1, bitorder="little")
        unp = unp.reshape(nQb, nKb, bq, W * 32).astype(bool)
        padded = np.zeros((nQb * bq, nKb * bk), bool); padded[:Sq, :Skv] = ok
        tiles = padded.reshape(nQb, bq, nKb, bk).transpose(0, 2, 1, 3)
        part = cls == 1
        assert part.any(), f"trial {trial} has no PARTIAL tile"
        assert np.array_equal(unp[..., :bk][part], tiles[part]), f"partial bits {trial}"
        assert not unp[..., bk:].any(), f"bits past the tile width {trial}"
        assert not unp[~part].any(), f"bits on a non-PARTIAL tile {trial}"
    # one allowed pair: exactly one word holds exactly one bit
    ok = np.zeros((70, 90), bool); ok[37, 77] = True
    bits = ora.partial_bits(ok, 32, 64)
    want = np.zeros_like(bits); want[1, 1, 5, 0] = np.uint32(1 << 13)
    assert np.array_equal(bits, want), "single pair bit"


ALL_PINS = [pin_mask_value_constant, pin_finite_mask_equivalence, pin_bruteforce, pin_sdpa,
            pin_closed_forms, pin_softcap, pin_merge, pin_chunked_equals_full, pin_sink_once,
            pin_gqa_repeat, pin_packed_docs, pin_ring_offsets, pin_block_mask, pin_dense_mask,
            pin_dense_chunked, pin_partial_bits]


# ---------------------------------------------------------------------------- backward
def _torch_forward(q, k, v, scale, ok, cap, sinks):
    """The forward written in torch (float64) for autograd: [B,Sq,H,D] layouts, ok [B,Sq,Skv].
    Masked pairs are dropped with torch.where (no -inf enters exp), so rows with nothing
    allowed give zeros without NaN."""
    H, Hkv = q.shape[2], k.shape[2]
    kr = k.repeat_interleave(H // Hkv, dim=2)
    vr = v.repeat_interleave(H // Hkv, dim=2)
    s = scale * torch.matmul(q.permute(0, 2, 1, 3), kr.permute(0, 2, 3, 1))      # [B,H,Sq,Skv]
    if cap is not None:
        s = cap * torch.tanh(s / cap)
    okb = ok[:, None].expand_as(s)
    m = torch.where(okb, s, torch.full_like(s, -math.inf)).amax(dim=-1, keepdim=True)
    if sinks is not None:
        m = torch.maximum(m, sinks[None, :, None, None].expand_as(m))
    m = torch.where(torch.isfinite(m), m, torch.zeros_like(m)).detach()
    e = torch.where(okb, torch.exp(s - m), torch.zeros_like(s))
    z = e.sum(dim=-1, keepdim=True)
    if sinks is not None:
        z = z + torch.exp(sinks[None, :, None, None] - m)
    p = e / torch.where(z > 0, z, torch.ones_like(z))
    return torch.matmul(p, vr.permute(0, 2, 1, 3)).permute(0, 2, 1, 3)


def pin_bwd_autograd(ora):
    """Backward = torch autograd of an independent torch forward (float64), with GQA, caps,
    sinks, segments with padding, shuffled positions, dense masks and empty rows."""
    rng = np.random.default_rng(26)
    for trial in range(10):
        B, Hkv = 1 + trial % 2, int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2, 3]))
        Sq, Skv, D = int(rng.integers(5, 40)), int(rng.integers(5, 40)), int(rng.choice([4, 8]))
        segs = trial >= 5
        q, k, v, qp, kp, qs, ks = _rand_problem(rng, B, Sq, Skv, H, Hkv, D, segs=segs,
                                                shuffle_pos=trial % 3 == 1, pad=segs)
        causal = trial % 4 != 3
        cap = 2.5 if trial % 2 else None
        sinks = rng.standard_normal(H) if trial % 3 != 2 else None
        dense = (rng.random((Sq, Skv)) < 0.7) if trial in (2, 5, 6, 9) else None
        if dense is not None:
            dense[Sq // 2] = False                               # an empty row
        ok = np.stack([ora.allowed(qp[b], kp[b], None if qs is None else qs[b], None if ks is None else ks[b],
                                   causal, dense) for b in range(B)])
        dout = rng.standard_normal(q.shape)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
        ts = None if sinks is None else torch.from_numpy(sinks).requires_grad_()
        o = _torch_forward(tq, tk, tv, 0.4, torch.from_numpy(ok), cap, ts)
        (o * torch.from_numpy(dout)).sum().backward()
        dq, dk, dv, dsk = ora.attention_bwd(q, k, v, dout, scale=0.4, q_pos=qp, kv_pos=kp, q_seg=qs,
                                            kv_seg=ks, causal=causal, softcap=cap, sinks=sinks, dense=dense)
        _close(dq, tq.grad.numpy(), 1e-10, f"autograd dq {trial}")
        _close(dk, tk.grad.numpy(), 1e-10, f"autograd dk {trial}")
        _close(dv, tv.grad.numpy(), 1e-10, f"autograd dv {trial}")
        if sinks is not None:
            _close(dsk, ts.grad.numpy(), 1e-10, f"autograd dsinks {trial}")
        assert np.abs(dq).max() > 0 and np.abs(dk).max() > 0


def pin_bwd_finite_differences(ora):
    """Central differences of L = sum(out * dout) through the oracle's own (pinned) forward."""
    rng = np.random.default_rng(27)
    B, Sq, Skv, H, Hkv, D = 1, 4, 5, 2, 1, 3
    q, k, v, qp, kp, _, _ = _rand_problem(rng, B, Sq, Skv, H, Hkv, D, shuffle_pos=True)
    sinks = rng.standard_normal(H)
    dout = rng.standard_normal(q.shape)
    kw = dict(scale=0.6, q_pos=qp, kv_pos=kp, causal=True, softcap=1.5)
    loss = lambda q_, k_, v_, s_: float(np.sum(ora.attention(q_, k_, v_, sinks=s_, **kw)[0] * dout))
    dq, dk, dv, dsk = ora.attention_bwd(q, k, v, dout, sinks=sinks, **kw)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("sinks", sinks, dsk)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps; xm[idx] -= eps
            args_p = [q, k, v, sinks]; args_m = [q, k, v, sinks]
            pos = ("q", "k", "v", "sinks").index(name)
            args_p[pos], args_m[pos] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        _close(g, num, 1e-7, f"finite differences d{name}")


def pin_bwd_chunked_and_gqa(ora):
    """Ring backward (chunk terms against the final out / lse, summed) = whole-KV backward, the
    sink counted once; GQA gradients = repeated-KV gradients summed over each group."""
    rng = np.random.default_rng(28)
    for trial in range(4):
        B, Sq, H, Hkv, D = 1 + trial % 2, 18 + trial, 4, 2, 6
        Skv = int(rng.integers(30, 50))
        q, k, v, qp, kp, qs, ks = _rand_problem(rng, B, Sq, Skv, H, Hkv, D, segs=trial >= 2, pad=trial >= 2)
        cap = 3.0 if trial % 2 else None
        sinks = rng.standard_normal(H)
        dense = rng.random((Sq, Skv)) < 0.8 if trial == 3 else None
        dout = rng.standard_normal(q.shape)
        cuts = np.sort(rng.choice(np.arange(1, Skv), size=2, replace=False))
        bounds = [(0, int(cuts[0])), (int(cuts[0]), int(cuts[1])), (int(cuts[1]), Skv)]
        kw = dict(scale=0.5, q_pos=qp, kv_pos=kp, q_seg=qs, kv_seg=ks, softcap=cap, sinks=sinks, dense=dense)
        ref = ora.attention_bwd(q, k, v, dout, **kw)
        got = ora.chunked_bwd(q, k, v, dout, bounds=bounds, **kw)
        for name, a, b_ in zip(("dq", "dk", "dv", "dsinks"), got, ref):
            _close(a, b_, 1e-11, f"chunked {name} {trial}")
    q, k, v, qp, kp, qs, ks = _rand_problem(rng, 1, 20, 26, 6, 2, 4, segs=True, pad=True)
    dout = rng.standard_normal(q.shape)
    kw = dict(scale=0.5, q_pos=qp, kv_pos=kp, q_seg=qs, kv_seg=ks, softcap=2.0, sinks=rng.standard_normal(6))
    g1 = ora.attention_bwd(q, k, v, dout, **kw)
    g2 = ora.attention_bwd(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), dout, **kw)
    _close(g1[0], g2[0], 1e-12, "gqa dq")
    _close(g1[1], g2[1].reshape(1, 26, 2, 3, 4).sum(axis=3), 1e-12, "gqa dk")
    _close(g1[2], g2[2].reshape(1, 26, 2, 3, 4).sum(axis=3), 1e-12, "gqa dv")
    _close(g1[3], g2[3], 1e-12, "gqa dsinks")


def pin_bwd_dq_rows(ora):
    """The query gradient of a sample of rows = torch autograd of the independent torch forward
    over all rows, read at those rows (GQA, caps, sinks, segments with padding, shuffled
    positions, dense masks with an empty row)."""
    rng = np.random.default_rng(29)
    for trial in range(8):
        B, Hkv = 1 + trial % 2, int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([2, 3]))
        Sq, Skv, D = int(rng.integers(8, 40)), int(rng.integers(5, 40)), int(rng.choice([4, 8]))
        segs = trial >= 4
        q, k, v, qp, kp, qs, ks = _rand_problem(rng, B, Sq, Skv, H, Hkv, D, segs=segs,
                                                shuffle_pos=trial % 3 == 1, pad=segs)
        causal = trial % 4 != 3
        cap = 1.7 if trial % 2 == 0 else None
        sinks = rng.standard_normal(H) if trial % 3 != 2 else None
        dense = (rng.random((Sq, Skv)) < 0.7) if trial in (1, 5) else None
        if dense is not None:
            dense[Sq // 3] = False
        ok = np.stack([ora.allowed(qp[b], kp[b], None if qs is None else qs[b], None if ks is None else ks[b],
                                   causal, dense) for b in range(B)])
        dout = rng.standard_normal(q.shape)
        tq = torch.from_numpy(q).requires_grad_()
        o = _torch_forward(tq, torch.from_numpy(k), torch.from_numpy(v), 0.45, torch.from_numpy(ok), cap,
                           None if sinks is None else torch.from_numpy(sinks))
        (o * torch.from_numpy(dout)).sum().backward()
        rows = np.sort(rng.choice(Sq, size=max(1, Sq // 3), replace=False))
        got = ora.attention_dq(q[:, rows], k, v, dout[:, rows], scale=0.45, q_pos=qp[:, rows], kv_pos=kp,
                               q_seg=None if qs is None else qs[:, rows], kv_seg=ks, causal=causal, softcap=cap,
                               sinks=sinks, dense=None if dense is None else dense[rows])
        _close(got, tq.grad.numpy()[:, rows], 1e-10, f"dq rows {trial}")
        assert np.abs(got).max() > 0


ALL_PINS += [pin_bwd_autograd, pin_bwd_finite_differences, pin_bwd_chunked_and_gqa, pin_bwd_dq_rows]
