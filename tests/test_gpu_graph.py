"""ring_attn_fwd_1gpu under HIP graph capture.

The ring forward makes no allocation, host synchronisation or memset: every step is a kernel
launch on the caller's stream into the caller's workspace, so a caller can capture it in a graph
and replay it. Each case captures one call, then replays the graph three times with other eager
work on the same stream in between (the outputs refilled with NaN, and the ring run on other
inputs into other buffers), and checks every replay bit for bit against an eager call on the same
inputs. The cases cover the kernel's instantiations: repacked V (the 32k ring's path), packed
documents (bits), a dense mask read over all keys, and a split ring with a soft cap and sinks.
The no-allocation entry point, whose workspace is the GPU's static scratch, is captured the same
way on two of them."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import ring_attention_merge_amd as ram
from ring_attention_merge_amd import workloads as wl
from gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = {
    # Sq * H / Hkv = 32768: the ring repacks V and reads it with row reads
    "packed_v_causal": dict(B=1, H=8, Hkv=2, Sq=8192, chunk=512, n=3, q_shard=-1, causal=True, cap=None,
                            sinks=False, feature="plain"),
    "packed_docs": dict(B=2, H=4, Hkv=4, Sq=1024, chunk=1024, n=1, q_shard=-1, causal=True, cap=None,
                        sinks=False, feature="docs"),
    "dense_shard": dict(B=1, H=4, Hkv=2, Sq=640, chunk=320, n=3, q_shard=1, causal=True, cap=None,
                        sinks=False, feature="dense"),
    # few q tile rows: the ring splits each row's visits over two workgroups, merged at the end
    "split_cap_sinks": dict(B=1, H=2, Hkv=1, Sq=512, chunk=256, n=4, q_shard=2, causal=True, cap=30.0,
                            sinks=True, feature="plain"),
}


def _setup(name: str, c: dict, seed: int):
    docs = (64, 512, 0.05) if c["feature"] == "docs" else None
    w = wl.make(f"graph_{name}_{seed}", B=c["B"], H=c["H"], Hkv=c["Hkv"], Sq=c["Sq"], chunk=c["chunk"],
                n_chunks=c["n"], D=128, dtype="bf16", causal=c["causal"], softcap=c["cap"],
                with_sinks=c["sinks"], q_shard=c["q_shard"], docs=docs, seed=seed)
    dense = None
    if c["feature"] == "dense":
        rng = np.random.default_rng(seed)
        dense = wl.dense_mask(rng, w.Sq, c["chunk"] * c["n"], q_offset=w.q_pos_base, window=96, n_global=4,
                              block=64)
    d = ram.Desc(B=w.B, Sq=w.Sq, Skv=c["chunk"], H=w.H, Hkv=w.Hkv, D=128, dtype=ram.RAM_BF16, scale=w.scale,
                 softcap=w.softcap or 0.0, causal=w.causal)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)
    src = ram.MaskSrc(q_pos=t(w.q_pos), kv_pos=t(w.kv_pos), q_seg=t(w.q_seg), kv_seg=t(w.kv_seg),
                      dense=None if dense is None else torch.from_numpy(dense).to(DEV),
                      dense_chunk_step=c["chunk"] if dense is not None else 0)
    io = dict(q=w.q.to(DEV), k=w.k.to(DEV), v=w.v.to(DEV), sinks=None if w.sinks is None else w.sinks.to(DEV),
              out=torch.empty(w.B, w.Sq, w.H, 128, dtype=torch.bfloat16, device=DEV),
              lse=torch.empty(w.B, w.H, w.Sq, device=DEV),
              ws=torch.empty(max(1, ram.ring_attn_workspace_bytes(d, c["n"], src)), dtype=torch.uint8, device=DEV))
    return d, src, io


def _call(d, src, c, io):
    ram.ring_attn_fwd_1gpu(d, c["n"], c["q_shard"], io["q"], io["k"], io["v"], src, io["sinks"], io["out"],
                           io["lse"], io["ws"])


@pytest.mark.parametrize("name", list(CASES))
def test_ring_forward_graph_replays(name):
    c = CASES[name]
    say(f"graph capture: {name} {c}")
    d, src, io = _setup(name, c, 4100)
    d2, src2, io2 = _setup(name, c, 4101)   # other inputs for the eager work between replays
    _call(d, src, c, io)
    torch.cuda.synchronize()
    out_ref, lse_ref = io["out"].clone(), io["lse"].clone()
    assert torch.isfinite(out_ref.float()).all()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        _call(d, src, c, io)
    torch.cuda.synchronize()
    for rep in range(3):
        io["out"].fill_(float("nan"))
        io["lse"].fill_(float("nan"))
        g.replay()
        _call(d2, src2, c, io2)
        torch.cuda.synchronize()
        assert torch.equal(io["out"], out_ref), f"{name}: replay {rep} output differs from the eager call"
        assert torch.equal(io["lse"], lse_ref), f"{name}: replay {rep} lse differs from the eager call"
    say(f"graph capture: {name} 3 replays bit-identical to the eager call")


@pytest.mark.parametrize("name", ["packed_v_causal", "split_cap_sinks"])
def test_noalloc_graph_replays(name):
    """ring_attn_fwd_1gpu_noalloc, the entry point for callers that cannot allocate (code under
    graph capture among them), captured in a graph and replayed three times with other eager
    calls of it in between (they share the GPU's static scratch, one at a time on the stream):
    every replay bit-identical to the eager call."""
    c = CASES[name]
    say(f"graph capture (no-alloc entry point): {name} {c}")
    d, src, io = _setup(name, c, 4200)
    d2, src2, io2 = _setup(name, c, 4201)

    def call(d_, src_, io_):
        ram.ring_attn_fwd_1gpu_noalloc(d_, c["n"], c["q_shard"], io_["q"], io_["k"], io_["v"], src_, io_["sinks"],
                                       io_["out"], io_["lse"])

    call(d, src, io)
    torch.cuda.synchronize()
    out_ref, lse_ref = io["out"].clone(), io["lse"].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        call(d, src, io)
    torch.cuda.synchronize()
    for rep in range(3):
        io["out"].fill_(float("nan"))
        io["lse"].fill_(float("nan"))
        g.replay()
        call(d2, src2, io2)
        torch.cuda.synchronize()
        assert torch.equal(io["out"], out_ref), f"{name}: no-alloc replay {rep} output differs from the eager call"
        assert torch.equal(io["lse"], lse_ref), f"{name}: no-alloc replay {rep} lse differs from the eager call"
    say(f"graph capture (no-alloc entry point): {name} 3 replays bit-identical to the eager call")
