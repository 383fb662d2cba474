"""Helpers for the GPU parity tests: run the HIP path through the binding and
compare with the float64 oracle at the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import ring_attention_merge_amd as ram

# Tolerances: output max-abs 2e-2 (bf16 inputs) / 1e-4 (fp32 inputs), lse 1e-3;
# rows the oracle leaves empty must be exactly (0, -inf).
OUT_TOL = {"bf16": 2e-2, "f32": 1e-4}
LSE_TOL = 1e-3


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def dtype_code(wl):
    return ram.RAM_BF16 if wl.dtype == "bf16" else ram.RAM_F32


def mask_src(wl, dev="cuda"):
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    return ram.MaskSrc(q_pos=t(wl.q_pos), kv_pos=t(wl.kv_pos), q_seg=t(wl.q_seg), kv_seg=t(wl.kv_seg))


def ring_desc(wl):
    return ram.Desc(B=wl.B, Sq=wl.Sq, Skv=wl.chunk, H=wl.H, Hkv=wl.Hkv, D=wl.D, dtype=dtype_code(wl),
                    scale=wl.scale, softcap=wl.softcap or 0.0, causal=wl.causal)


def run_ring(wl, dev="cuda", poison=True):
    """ring_attn_fwd_1gpu on a workload; returns (out float32 CPU, lse CPU)."""
    d = ring_desc(wl)
    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    sinks = None if wl.sinks is None else wl.sinks.to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(wl.B, wl.H, wl.Sq, dtype=torch.float32, device=dev)
    if poison:
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
    src = mask_src(wl, dev)
    ws = torch.empty(max(1, ram.ring_attn_workspace_bytes(d, wl.n_chunks, src)), dtype=torch.uint8, device=dev)
    ram.ring_attn_fwd_1gpu(d, wl.n_chunks, wl.q_shard, q, k, v, src, sinks, out, lse, ws)
    torch.cuda.synchronize()
    return out.float().cpu(), lse.cpu()


def oracle_ref(wl, rows=None):
    q, k, v, sinks = wl.as_f64()
    qp, kp = wl.positions()
    return oracle.attention(q, k, v, scale=wl.scale, q_pos=qp, kv_pos=kp, q_seg=wl.q_seg, kv_seg=wl.kv_seg,
                            causal=wl.causal, softcap=wl.softcap, sinks=sinks, rows=rows)


def compare(out, lse, ref_out, ref_lse, dtype, what, rows=None):
    """Max-abs parity; exact (0, -inf) where the oracle row is empty."""
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    if rows is not None:
        out = out[:, rows]
        lse = lse[:, :, rows]
    assert out.shape == ref_out.shape and lse.shape == ref_lse.shape, (out.shape, ref_out.shape)
    assert not np.isnan(out).any(), f"{what}: NaN in out (unwritten or bad arithmetic)"
    assert not np.isnan(lse).any(), f"{what}: NaN in lse"
    empty = ref_lse == -np.inf                          # [B,H,R]
    assert np.array_equal(lse == -np.inf, empty), f"{what}: -inf rows differ"
    e4 = np.transpose(empty, (0, 2, 1))                 # [B,R,H]
    assert np.all(out[e4] == 0), f"{what}: empty rows not zero"
    err_o = float(np.max(np.abs(out - ref_out))) if out.size else 0.0
    fin = ~empty
    err_l = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    say(f"{what}: out max err {err_o:.3e} (tol {OUT_TOL[dtype]:.0e}), lse max err {err_l:.3e}")
    assert err_o <= OUT_TOL[dtype], f"{what}: out err {err_o}"
    assert err_l <= LSE_TOL, f"{what}: lse err {err_l}"
    return err_o, err_l


def ring_by_chunks(d, n, r, q, k, v, src, sinks, dev="cuda"):
    """The ring of ring_attn_fwd_1gpu(d, n, r, ...) as a loop of attn_fwd_chunk calls in ring
    order (WRITE on the first visit with the sinks, MERGE after), each chunk's block mask built
    on its own; returns the float32 (out, lse) on the device. Key positions, segment IDs and the
    dense-mask columns travel with their chunk."""
    C = d.Skv
    bq, bk = ram.kernel_tile(d.dtype, d.D)
    kv_total = n * C
    out = torch.empty(d.B, d.Sq, d.H, d.D, dtype=torch.float32, device=dev)
    lse = torch.empty(d.B, d.H, d.Sq, dtype=torch.float32, device=dev)
    q_base = src.q_pos_base + (r * d.Sq if r >= 0 else 0)
    kvm = src.kv_meta_stride_b or kv_total
    step = src.dense_chunk_step
    ld = src.dense_ld or (C + (n - 1) * step)
    esz = k.element_size()
    for t in range(n):
        c = (r - t) % n if r >= 0 else t
        dc = ram.Desc(**{**d.__dict__, "block_q": bq, "block_kv": bk, "kv_stride_b": kv_total * d.Hkv * d.D})
        sc = ram.MaskSrc(q_pos=src.q_pos, q_pos_base=q_base, q_seg=src.q_seg, q_meta_stride_b=src.q_meta_stride_b,
                         kv_pos=None if src.kv_pos is None else src.kv_pos.view(-1)[c * C:],
                         kv_pos_base=src.kv_pos_base + c * C,
                         kv_seg=None if src.kv_seg is None else src.kv_seg.view(-1)[c * C:],
                         kv_meta_stride_b=kvm,
                         dense=None if src.dense is None else src.dense.view(-1)[c * step:],
                         dense_ld=ld if src.dense is not None else 0)
        bm = ram.alloc_block_mask(dc, device=dev, with_bits=True)
        ram.build_block_mask(dc, sc, bm)
        kc = k.view(-1)[c * C * d.Hkv * d.D:]
        vc = v.view(-1)[c * C * d.Hkv * d.D:]
        ram.attn_fwd_chunk(dc, q, kc, vc, sc, bm, sinks if t == 0 else None, 0 if t == 0 else 1, out, lse)
    assert esz in (2, 4)
    return out, lse


def ring_splits(d, n) -> bool:
    """Whether ring_attn_fwd_1gpu splits each row of q tiles' visits over two workgroups (the
    bf16 D = 128 kernel with fewer rows than compute units)."""
    bq, _ = ram.kernel_tile(d.dtype, d.D)
    return d.dtype == ram.RAM_BF16 and d.D == 128 and n >= 2 and d.B * d.H * (-(-d.Sq // bq)) < 512
