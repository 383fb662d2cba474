"""The MFMA rate probe that the bench reports beside the published peak: it runs, zero operands
give zero checksums, random ones finite and non-zero ones."""
import pytest
import torch

import ring_attention_merge_amd as ram

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs():
    out = torch.full((4 * 512,), float("nan"), device="cuda")
    ram.mfma_probe(4, 3, 0, out)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out))
    ram.mfma_probe(4, 3, 1, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (out != 0).any()


def test_kernel_events_time_the_ring():
    """Events set with set_kernel_events bracket the ring's attention launch: they measure a positive
    time no longer than the whole call's, and the result is the same as without them."""
    from ring_attention_merge_amd import workloads as wl
    w = wl.c2_ring_shard(Sq=512, H=2, seed=41)
    d = ram.Desc(B=w.B, Sq=w.Sq, Skv=w.chunk, H=w.H, Hkv=w.Hkv, D=w.D, scale=w.scale, causal=True)
    q, k, v = w.q.cuda(), w.k.cuda(), w.v.cuda()
    src = ram.MaskSrc()
    ws = torch.empty(ram.ring_attn_workspace_bytes(d, w.n_chunks), dtype=torch.uint8, device="cuda")
    out0, out1 = torch.empty_like(q), torch.empty_like(q)
    lse0, lse1 = (torch.empty(w.B, w.H, w.Sq, device="cuda") for _ in range(2))
    ram.ring_attn_fwd_1gpu(d, w.n_chunks, w.q_shard, q, k, v, src, None, out0, lse0, ws)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    ram.set_kernel_events(a, b)
    try:
        ram.ring_attn_fwd_1gpu(d, w.n_chunks, w.q_shard, q, k, v, src, None, out1, lse1, ws)
    finally:
        ram.set_kernel_events()
    c1.record()
    torch.cuda.synchronize()
    assert 0 < a.elapsed_time(b) <= c0.elapsed_time(c1)
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)
