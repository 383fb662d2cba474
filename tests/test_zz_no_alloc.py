"""ring_attn_fwd_1gpu_noalloc, the ring with the library's static per-GPU scratch instead of a
workspace, gives exactly what ring_attn_fwd_1gpu gives with a workspace (same kernels, same
launches): on two calls in a row, the second with a smaller input on the scratch the first one
left behind, plus a third with stored tile bits."""
from __future__ import annotations

import pytest
import torch

import ring_attention_merge_amd as ram
from ring_attention_merge_amd import workloads as wl

from gpu_util import mask_src, ring_desc, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(w):
    d = ring_desc(w)
    src = mask_src(w, DEV)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    sinks = None if w.sinks is None else w.sinks.to(DEV)
    res = []
    for noalloc in (False, True):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((w.B, w.H, w.Sq), float("nan"), device=DEV)
        if noalloc:
            ram.ring_attn_fwd_1gpu_noalloc(d, w.n_chunks, w.q_shard, q, k, v, src, sinks, out, lse)
        else:
            ws = torch.empty(ram.ring_attn_workspace_bytes(d, w.n_chunks, src), dtype=torch.uint8, device=DEV)
            ram.ring_attn_fwd_1gpu(d, w.n_chunks, w.q_shard, q, k, v, src, sinks, out, lse, ws)
        torch.cuda.synchronize()
        res.append((out.cpu(), lse.cpu()))
    return res


def test_noalloc_ring_equals_workspace_ring():
    cases = [
        # a split ring (its second half's running state in the scratch too), 4 chunks, shard 3
        wl.c2_ring_shard(Sq=2048, H=8, seed=301),
        # smaller, on the scratch the first call left: GQA, soft cap, sinks, ragged chunks
        wl.make("small_cap_sinks", B=2, H=4, Hkv=2, Sq=300, chunk=200, n_chunks=3, D=128, softcap=30.0,
                with_sinks=True, q_shard=1, seed=302),
        # packed documents: the PARTIAL tiles' bits stored in the scratch as well
        wl.make("small_docs", B=2, H=2, Hkv=2, Sq=640, chunk=320, n_chunks=2, D=128, docs=(40, 300, 0.05),
                seed=303),
    ]
    for w in cases:
        say(f"no-alloc ring {w.name}: B={w.B} H={w.H} Sq={w.Sq} chunks {w.n_chunks} x {w.chunk}")
        (o1, l1), (o2, l2) = _both(w)
        assert not torch.isnan(o1.float()).any() and not torch.isnan(l1).any()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{w.name}: no-alloc ring differs from the workspace ring"
