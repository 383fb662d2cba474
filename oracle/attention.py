"""Plain float64 attention, element mask and LSE merge. TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline may use this.

Sources (the pages):
  [ring]  ejkernel module source page "ejkernel.kernels._pallas.tpu.ring_attention._ring_splash":
          _update_out_and_lse (the merge), _ring_attention_forward (causal
          predicate on shifted q ids, sinks only on the first ring step, fp32
          accumulators, output cast to the q dtype).
  [api]   ejkernel API page for the same module: the default mask_value.
  [kvax]  "Kvax: Flash Attention for JAX" page: flash_attention and
          create_attention_mask arguments ([B,S,H,D] layouts, positions and
          segment IDs, padding segment, scale).
  [bwd]   the same page's _ring_attention_backward: the chunk backward per ring
          step against the final out and logsumexp, gradients summed.
  [make]  the ring-splash page's make_ring_attention: a two-dimensional
          boolean mask over (query, key) given by the caller, turned into the
          block mask and partial-block contents of MaskInfo.

The method reaches, up to rounding order, ordinary masked softmax attention
over the full key set, so ``attention`` is that definition written out: it
builds every score, masks it, and normalises, with no tiling and no online
softmax. Readings of points the pages leave open (see the project design notes):
  * a sink is one extra logit per query head in the normaliser with no value
    row; it is neither scaled nor capped;
  * masked pairs are excluded exactly (weight 0); a row with nothing allowed
    gives out = 0 and lse = -inf (lse = sink with a sink);
  * the soft cap is cap * tanh(s / cap) on the scaled logit s = scale * q.k;
  * causal means kv_pos <= q_pos; segments must be equal and not padding;
  * a dense mask is one [Sq, Skv] boolean array shared by every batch row and
    head; a pair takes part only if the dense mask, the causal test and the
    segment test all allow it (the pages' ring uses the dense mask on its
    non-causal path, where it and the segment IDs both apply);
  * in the chunked fold, chunk c reads the dense mask's columns from a start
    column of its own: the chunk's first key for one mask over the whole KV,
    or 0 for every chunk to reuse one local mask at each step (what the
    pages' non-causal ring does with its fixed mask info);
  * query head h reads KV head h // (H / Hkv);
  * lse is the natural log, laid out [B, H, Sq].
"""
from __future__ import annotations

import numpy as np

# The finite mask value printed on the [api] page, equal to -0.7 * float32 max.
DEFAULT_MASK_VALUE = -2.381976426469702e38
# Padding segment ID ([kvax] names the constant without a value; -1 is the reading).
PAD_SEGMENT_ID = -1


def allowed(q_pos, kv_pos, q_seg=None, kv_seg=None, causal=True, dense=None):
    """Element mask for one batch row: [Sq, Skv] bool.

    [ring] _ring_attention_forward: the causal mask keeps a key when the query
    id is >= the key id, ids being positions shifted by the ring offsets.
    [kvax] flash_attention: tokens attend within their own segment; padding
    tokens carry the padding segment ID and take part in nothing.
    [make] make_ring_attention: ``dense`` [Sq, Skv] (nonzero = allowed) is
    the caller's two-dimensional mask; it further restricts the pairs.
    """
    q_pos = np.asarray(q_pos)
    kv_pos = np.asarray(kv_pos)
    ok = np.ones((q_pos.shape[0], kv_pos.shape[0]), dtype=bool)
    if dense is not None:
        dense = np.asarray(dense)
        if dense.shape != ok.shape:
            raise ValueError(f"dense mask of shape {dense.shape}, expected {ok.shape}")
        ok &= dense != 0
    if causal:
        ok &= kv_pos[None, :] <= q_pos[:, None]
    if q_seg is not None:
        q_seg = np.asarray(q_seg)
        kv_seg = np.asarray(kv_seg)
        ok &= q_seg[:, None] == kv_seg[None, :]
        ok &= (q_seg != PAD_SEGMENT_ID)[:, None]
    return ok


def attention(q, k, v, *, scale, q_pos, kv_pos, q_seg=None, kv_seg=None, causal=True,
              softcap=None, sinks=None, dense=None, rows=None, row_block=512):
    """Masked softmax attention in float64 from the full score matrix.

    q [B,Sq,H,D], k and v [B,Skv,Hkv,D]; positions [B,Sq] / [B,Skv]; segment
    IDs the same or None; sinks [H] or None; ``dense`` [Sq, Skv] or None, one
    mask for every batch row and head. ``rows`` restricts the query rows
    computed (for sampled checks). Returns out [B,R,H,D] and lse [B,H,R] in
    float64, R = Sq or len(rows).

    For query row i of head h (KV head g = h // (H / Hkv)):
        s_ij  = scale * sum_d q[i,h,d] k[j,g,d];   s_ij = cap*tanh(s_ij/cap) if capped
        Z_i   = sum over allowed j of exp(s_ij)  (+ exp(sink_h) with sinks)
        out_i = sum over allowed j of exp(s_ij) v[j,g,:] / Z_i    (0 if Z_i = 0)
        lse_i = ln Z_i                                            (-inf if Z_i = 0)
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Sq, H, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    G = H // Hkv
    row_idx = np.arange(Sq) if rows is None else np.asarray(rows, np.int64)
    R = row_idx.shape[0]
    out = np.zeros((B, R, H, D))
    lse = np.full((B, H, R), -np.inf)
    for b in range(B):
        for start in range(0, R, row_block):
            r = row_idx[start:start + row_block]
            ok = allowed(np.asarray(q_pos)[b, r], np.asarray(kv_pos)[b],
                         None if q_seg is None else np.asarray(q_seg)[b, r],
                         None if kv_seg is None else np.asarray(kv_seg)[b], causal,
                         None if dense is None else np.asarray(dense)[r])
            for h in range(H):
                g = h // G
                s = scale * (q[b, r, h, :] @ k[b, :, g, :].T)
                if softcap is not None:
                    s = softcap * np.tanh(s / softcap)
                s = np.where(ok, s, -np.inf)
                if sinks is not None:
                    s = np.concatenate([s, np.full((len(r), 1), float(sinks[h]))], axis=1)
                m = s.max(axis=1)
                m_safe = np.where(np.isfinite(m), m, 0.0)
                e = np.exp(s - m_safe[:, None])
                z = e.sum(axis=1)
                num = e[:, :Skv] @ v[b, :, g, :]
                nz = z > 0
                o = np.zeros_like(num)
                o[nz] = num[nz] / z[nz, None]
                out[b, start:start + len(r), h, :] = o
                lse[b, h, start:start + len(r)] = np.where(nz, m_safe + np.log(np.where(nz, z, 1.0)),
                                                           -np.inf)
    return out, lse


def merge(out, lse, block_out, block_lse):
    """Fold one chunk's (block_out, block_lse) into the running (out, lse), float64.

    [ring] _update_out_and_lse: a row whose running lse is -inf takes the
    block's values; otherwise, with x = block_lse - lse, the output moves
    toward the block's by the weight sigmoid(x) and lse grows by softplus(x).
    Layouts: out [B,Sq,H,D], lse [B,H,Sq].
    """
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    block_out = np.asarray(block_out, np.float64)
    block_lse = np.asarray(block_lse, np.float64)
    is_first = lse == -np.inf
    with np.errstate(invalid="ignore", over="ignore"):
        x = np.where(is_first, 0.0, block_lse - lse)      # lse = -inf rows use the block values
        sig = 1.0 / (1.0 + np.exp(-x))
        softplus = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
    w = np.transpose(sig, (0, 2, 1))[..., None]          # [B,H,Sq] -> [B,Sq,H,1]
    new_out = out - w * (out - block_out)
    new_lse = lse + softplus
    first4 = np.transpose(is_first, (0, 2, 1))[..., None]
    new_out = np.where(first4, block_out, new_out)
    new_lse = np.where(is_first, block_lse, new_lse)
    return new_out, new_lse


def chunked(q, k, v, *, scale, q_pos, kv_pos, bounds, order, q_seg=None, kv_seg=None,
            causal=True, softcap=None, sinks=None, dense=None, dense_col0=None, rows=None):
    """Attention per KV chunk, folded with ``merge`` in the given chunk order.

    [ring] _ring_attention_forward: the running state starts at out = 0,
    lse = -inf; each step attends to one KV chunk and merges it in; sinks
    enter only on the first step. ``bounds`` lists each chunk's [start, end)
    key range; ``order`` lists chunk indices in visiting order. Chunk segment
    IDs and positions travel with their keys. With a ``dense`` mask [Sq, n],
    chunk c reads its columns from ``dense_col0[c]`` on (default: the chunk's
    first key, i.e. one mask over the whole KV).
    """
    q = np.asarray(q, np.float64)
    B, Sq, H, D = q.shape
    R = Sq if rows is None else len(rows)
    acc = np.zeros((B, R, H, D))
    acc_lse = np.full((B, H, R), -np.inf)
    for t, c in enumerate(order):
        a, e = bounds[c]
        dense_c = None
        if dense is not None:
            c0 = a if dense_col0 is None else dense_col0[c]
            dense_c = np.asarray(dense)[:, c0:c0 + (e - a)]
        o_c, l_c = attention(q, np.asarray(k)[:, a:e], np.asarray(v)[:, a:e], scale=scale,
                             q_pos=q_pos, kv_pos=np.asarray(kv_pos)[:, a:e], q_seg=q_seg,
                             kv_seg=None if kv_seg is None else np.asarray(kv_seg)[:, a:e],
                             causal=causal, softcap=softcap, dense=dense_c,
                             sinks=sinks if t == 0 else None, rows=rows)
        acc, acc_lse = merge(acc, acc_lse, o_c, l_c)
    return acc, acc_lse


def attention_bwd(q, k, v, dout, *, scale, q_pos, kv_pos, q_seg=None, kv_seg=None, causal=True,
                  softcap=None, sinks=None, dense=None, out=None, lse=None, row_block=512):
    """Gradients of ``attention`` with respect to q, k, v and the sinks, in float64.

    [ring] _ring_attention_backward runs the chunk kernel's backward once per ring
    step with the final ``out`` and ``logsumexp`` as residuals and sums the chunk
    gradients. This function is the gradient of the forward defined above, written
    out from the full score matrix (no tiling): for query row i of head h and an
    allowed key j (KV head g),
        t_ij = tanh(s_ij / cap) with s_ij = scale * q_i.k_j;  u_ij = cap * t_ij  (u = s uncapped)
        p_ij = exp(u_ij - lse_i),      p_sink,i = exp(sink_h - lse_i)
        dp_ij = dout_i . v_j,          D_i = dout_i . out_i
        du_ij = p_ij (dp_ij - D_i),    ds_ij = du_ij (1 - t_ij^2)   (ds = du uncapped)
        dq_i  = scale * sum_j ds_ij k_j
        dk_j += scale * sum_i ds_ij q_i      (summed over the heads sharing KV head g)
        dv_j += sum_i p_ij dout_i            (likewise)
        dsink_h = - sum over batch rows and queries of p_sink,i * D_i
    ``out`` / ``lse`` default to this module's forward on the same inputs; passing
    the forward's stored results reproduces the pages' use of residuals. Rows with
    lse = -inf contribute nothing. Returns (dq, dk, dv, dsinks) with dsinks None
    when there are no sinks.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    B, Sq, H, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    G = H // Hkv
    if out is None or lse is None:
        out, lse = attention(q, k, v, scale=scale, q_pos=q_pos, kv_pos=kv_pos, q_seg=q_seg,
                             kv_seg=kv_seg, causal=causal, softcap=softcap, sinks=sinks, dense=dense)
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsinks = None if sinks is None else np.zeros(H)
    for b in range(B):
        for start in range(0, Sq, row_block):
            r = np.arange(start, min(Sq, start + row_block))
            ok = allowed(np.asarray(q_pos)[b, r], np.asarray(kv_pos)[b],
                         None if q_seg is None else np.asarray(q_seg)[b, r],
                         None if kv_seg is None else np.asarray(kv_seg)[b], causal,
                         None if dense is None else np.asarray(dense)[r])
            for h in range(H):
                g = h // G
                l = lse[b, h, r]
                live = np.isfinite(l)
                l_safe = np.where(live, l, 0.0)
                s = scale * (q[b, r, h, :] @ k[b, :, g, :].T)
                if softcap is not None:
                    t = np.tanh(s / softcap)
                    u = softcap * t
                else:
                    u = s
                p = np.where(ok & live[:, None], np.exp(u - l_safe[:, None]), 0.0)
                do = dout[b, r, h, :]
                dp = do @ v[b, :, g, :].T
                Drow = np.sum(do * out[b, r, h, :], axis=1)
                du = p * (dp - Drow[:, None])
                ds = du * (1.0 - t * t) if softcap is not None else du
                dq[b, r, h, :] = scale * (ds @ k[b, :, g, :])
                dk[b, :, g, :] += scale * (ds.T @ q[b, r, h, :])
                dv[b, :, g, :] += p.T @ do
                if sinks is not None:
                    ps = np.where(live, np.exp(float(sinks[h]) - l_safe), 0.0)
                    dsinks[h] -= float(np.sum(ps * Drow))
    return dq, dk, dv, dsinks


def attention_dq(q, k, v, dout, *, scale, q_pos, kv_pos, q_seg=None, kv_seg=None, causal=True,
                 softcap=None, sinks=None, dense=None):
    """The query gradient alone, for the query rows passed, in float64.

    [bwd] the chunk backward's dq term (its sum over the ring's chunks is the whole-KV
    gradient, see ``chunked_bwd``). The gradient of ``attention`` with respect to query row i depends only on that row
    and on every key, so a caller may pass a sample of rows (with their positions,
    segment IDs and dense-mask rows) to check a full-size result row by row. With the
    same notation as ``attention_bwd``:
        dq_i = scale * sum over allowed j of p_ij (dp_ij - D_i) (1 - t_ij^2) k_j
    where p_ij = exp(u_ij - lse_i), dp_ij = dout_i . v_j and D_i = dout_i . out_i, with
    (out_i, lse_i) from ``attention`` on the same rows (the sink, when given, enters only
    through lse_i and out_i). Returns dq with q's shape.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    B, Sq, H, D = q.shape
    Hkv = k.shape[2]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    per_kv = H // Hkv
    out, lse = attention(q, k, v, scale=scale, q_pos=q_pos, kv_pos=kv_pos, q_seg=q_seg, kv_seg=kv_seg,
                         causal=causal, softcap=softcap, sinks=sinks, dense=dense)
    grad = np.zeros_like(q)
    for b in range(B):
        keep = allowed(np.asarray(q_pos)[b], np.asarray(kv_pos)[b],
                       None if q_seg is None else np.asarray(q_seg)[b],
                       None if kv_seg is None else np.asarray(kv_seg)[b], causal,
                       None if dense is None else np.asarray(dense))
        for h in range(H):
            kv_h = h // per_kv
            logz = lse[b, h]
            seen = np.isfinite(logz)
            logits = scale * np.einsum("id,jd->ij", q[b, :, h, :], k[b, :, kv_h, :])
            tanh_t = None
            if softcap is not None:
                tanh_t = np.tanh(logits / softcap)
                logits = softcap * tanh_t
            prob = np.where(keep & seen[:, None], np.exp(logits - np.where(seen, logz, 0.0)[:, None]), 0.0)
            g_prob = np.einsum("id,jd->ij", dout[b, :, h, :], v[b, :, kv_h, :])
            delta = np.einsum("id,id->i", dout[b, :, h, :], out[b, :, h, :])
            g_logit = prob * (g_prob - delta[:, None])
            if tanh_t is not None:
                g_logit = g_logit * (1.0 - tanh_t ** 2)
            grad[b, :, h, :] = scale * np.einsum("ij,jd->id", g_logit, k[b, :, kv_h, :])
    return grad


def chunked_bwd(q, k, v, dout, *, scale, q_pos, kv_pos, bounds, q_seg=None, kv_seg=None, causal=True,
                softcap=None, sinks=None, dense=None, dense_col0=None):
    """The ring backward: per-chunk gradients against the final (out, lse), summed.

    [ring] _ring_attention_backward: every step runs the chunk backward with the
    final ``out`` and ``logsumexp`` of the whole ring as residuals; dq sums over the
    steps, dk and dv belong to the chunk they were computed on. The chunk terms
    are ``attention_bwd`` restricted to the chunk's keys with those residuals. The
    sink term does not depend on the keys and is taken once (reading: the gradient
    of a forward in which the sink enters once).
    """
    out, lse = chunked(q, k, v, scale=scale, q_pos=q_pos, kv_pos=kv_pos, bounds=bounds,
                       order=list(range(len(bounds))), q_seg=q_seg, kv_seg=kv_seg, causal=causal,
                       softcap=softcap, sinks=sinks, dense=dense, dense_col0=dense_col0)
    q = np.asarray(q, np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros(np.shape(k))
    dv = np.zeros(np.shape(v))
    dsinks = None
    for c, (a, e) in enumerate(bounds):
        dense_c = None
        if dense is not None:
            c0 = a if dense_col0 is None else dense_col0[c]
            dense_c = np.asarray(dense)[:, c0:c0 + (e - a)]
        dq_c, dk_c, dv_c, ds_c = attention_bwd(
            q, np.asarray(k)[:, a:e], np.asarray(v)[:, a:e], dout, scale=scale, q_pos=q_pos,
            kv_pos=np.asarray(kv_pos)[:, a:e], q_seg=q_seg,
            kv_seg=None if kv_seg is None else np.asarray(kv_seg)[:, a:e], causal=causal,
            softcap=softcap, sinks=sinks if c == 0 else None, dense=dense_c, out=out, lse=lse)
        dq += dq_c
        dk[:, a:e] = dk_c
        dv[:, a:e] = dv_c
        if ds_c is not None:
            dsinks = ds_c if dsinks is None else dsinks + ds_c
    return dq, dk, dv, dsinks
