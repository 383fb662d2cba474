#!/usr/bin/env python3
"""Throughput of the chunked (ring) attention forward on one MI355X.

A step is one ring_attn_fwd_1gpu call over one batch of synthetic input: the
block-mask build of every chunk and eight chunk launches of the attention
kernel (the first writes, the rest merge by LSE, the last also writes the bf16
result). The workload is
long-context causal attention: B=1, H=32 query heads over Hkv=8 KV heads,
32768 queries, 32768 keys in 8 sequential chunks of 4096, D=128, bf16 q, k
~ N(0,1) and v ~ U(-1,1). Inputs are resident in HBM before timing starts.

value: effective TFLOP/s = 4*D*H*(non-EMPTY 128x128 tiles over all chunks)*128^2
       divided by the step time. The tiles are counted here in numpy from the
       workload's positions, segment IDs and dense mask (not by the library);
       the line also says whether the library's own count agrees.
roofline: the attention kernel alone: the library records HIP events on the
       step's stream around its one attention launch in every timed step (the
       same window as the step time); achieved = its effective FLOPs / the
       median launch time, against the dense bf16 MFMA peak.
cpu_baseline: the float64 oracle on a bounded sample of query rows of the
       same workload (all heads, all keys), in pair FLOPs per second, with the
       host's cores and CPU model, and the full-size time extrapolated from
       the sample (labelled as such).

--backward times ring_attn_bwd_1gpu instead (out and lse from one forward
call before timing, dout ~ N(0,1) in bf16): value = 2.5x the forward's
effective FLOPs (five products per pair: S, dP, dV, dK, dQ) per second; the
roofline leg times each chunk's attn_bwd_chunk call (its dq and dk/dv
kernels) with HIP events, against the same FLOPs.

--workload c5dense runs the same shape with a dense two-dimensional mask over
all keys (ANDed with the causal test): the step then also classifies every
pair of the mask, the chunk kernel masks PARTIAL tiles from their stored bits,
and the line carries a `mask_builder` object (the builder alone over the whole
mask, against HBM bandwidth).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import ring_attention_merge_amd as ram  # noqa: E402
from ring_attention_merge_amd import workloads as wl  # noqa: E402

METRIC = "effective attention fwd TFLOP/s (unmasked tiles) and % bf16 MFMA peak, 1 GPU"
METRIC_BWD = "effective attention bwd TFLOP/s (unmasked tiles, 2.5x fwd FLOPs) and % bf16 MFMA peak, 1 GPU"
BWD_FLOP_FACTOR = 2.5
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
REF_TILE = 128                  # fixed reference tiling for effective FLOPs
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, published
KERNEL = "attn_fwd_bf16_alt"    # the bf16 D = 128 forward kernel the ring launches


def ring_kernel_name(cap: bool, bits: bool, split: bool, packed_v: bool) -> str:
    """The kernel instantiation a ring launch runs (soft cap, stored mask bits, split ring, V
    repacked for row reads)."""
    f = lambda x: str(bool(x)).lower()
    return f"{KERNEL}<{f(cap)}, {f(bits)}, {f(split)}, {f(packed_v)}>"


def ring_splits(w, bq: int) -> bool:
    """Whether the ring runs each row of q tiles as two half rings (the library does so when its
    rows of 128-row tiles give fewer than 512 workgroups)."""
    return w.n_chunks >= 2 and w.B * w.H * -(-w.Sq // bq) < 512


def ring_packs_v(w) -> bool:
    """Whether the ring reads V repacked for row reads (the library does so without a soft cap when
    Sq * H / Hkv >= 32768)."""
    return not w.softcap and w.Sq * (w.H // w.Hkv) >= 32768


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload(name: str):
    return {
        "c5": wl.c5_long_causal,
        "c4": wl.c4_gqa_cap_sinks,
        "c4mqa": lambda: wl.c4_gqa_cap_sinks(Hkv=1),
        "c3": wl.c3_packed_docs,
        "c2": wl.c2_ring_shard,
        "c5dense": wl.c5_dense,
    }[name]()


def dense_tensor(w, dev):
    return None if w.dense is None else torch.from_numpy(w.dense).to(dev)


def ring_chunk_src(w, c, dev, dense=None):
    """Mask source of chunk c of the ring (positions, segments and dense-mask columns travel
    with the chunk)."""
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    q_base = (w.q_shard * w.Sq if w.q_shard >= 0 else 0)
    kp = None if w.kv_pos is None else t(w.kv_pos[:, c * w.chunk:(c + 1) * w.chunk])
    ks = None if w.kv_seg is None else t(w.kv_seg[:, c * w.chunk:(c + 1) * w.chunk])
    dv = None if dense is None else dense.view(-1)[c * w.chunk:]   # column c*chunk, row stride Skv
    return ram.MaskSrc(q_pos=t(w.q_pos), kv_pos=kp, q_pos_base=q_base, kv_pos_base=c * w.chunk,
                       q_seg=t(w.q_seg), kv_seg=ks, dense=dv, dense_ld=w.Skv if dense is not None else 0)


def tile_counts(w, desc, dev, tile_q, tile_kv, dense=None):
    """Non-EMPTY tiles per chunk at (tile_q, tile_kv), from the library's block-mask builder."""
    counts = []
    for c in range(w.n_chunks):
        d = ram.Desc(**{**desc.__dict__, "block_q": tile_q, "block_kv": tile_kv})
        bm = ram.alloc_block_mask(d, device=dev)
        ram.build_block_mask(d, ring_chunk_src(w, c, dev, dense), bm)
        torch.cuda.synchronize()
        counts.append(int(bm.row_cnt[: d.B * bm.nQb].sum().item()))
    return counts


KERNEL_SOURCES = ("attn_fwd_alt.hip", "attn_common.h")   # what the ring's attention kernel is built from


def independent_tiles(w, T: int = REF_TILE):
    """Non-EMPTY TxT tiles per chunk, counted here in numpy from the workload's own arrays (no
    library code): a tile is non-EMPTY when one of its (query, key) pairs is allowed, i.e. the
    key's position is not past the query's (causal), both carry the same segment ID and it is not
    the padding ID, and the dense mask keeps the pair."""
    qp, kp = w.positions()
    nK = -(-w.chunk // T)
    rows = 8 * T
    counts = []
    for c in range(w.n_chunks):
        ks = slice(c * w.chunk, (c + 1) * w.chunk)
        n = 0
        for b in range(w.B):
            for r0 in range(0, w.Sq, rows):
                r1 = min(w.Sq, r0 + rows)
                ok = np.ones((r1 - r0, w.chunk), dtype=bool)
                if w.causal:
                    ok &= kp[b, ks][None, :] <= qp[b, r0:r1][:, None]
                if w.q_seg is not None:
                    qs = w.q_seg[b, r0:r1]
                    ok &= (qs[:, None] == w.kv_seg[b, ks][None, :]) & (qs != wl.PAD_SEGMENT_ID)[:, None]
                if w.dense is not None:
                    ok &= w.dense[r0:r1, ks] != 0
                rq = -(-(r1 - r0) // T) * T
                full = np.zeros((rq, nK * T), dtype=bool)
                full[: r1 - r0, : w.chunk] = ok
                n += int(full.reshape(rq // T, T, nK, T).any(axis=(1, 3)).sum())
        counts.append(n)
    return counts


def host_cpu():
    """Cores this process may run on and the CPU model (from /proc/cpuinfo)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return len(os.sched_getaffinity(0)), model


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "ring_attention_merge_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def recorded_bwd(workload: str, what: str, key: str):
    """A figure of the ring backward (the dq ring and the dk/dv launches) from the committed counter
    summary profiles/attn_bwd_<workload>_<what>.md, if it was taken on the current backward source
    (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"attn_bwd_{workload}_{what}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        line = line.strip().strip("`")
        if "=" in line and " " not in line.split("=", 1)[0]:
            k, v = line.split("=", 1)
            fields[k] = v.strip()
    h = hashlib.sha256()
    for f in ("attn_bwd.hip", "attn_common.h"):
        h.update(open(os.path.join(ROOT, "ring_attention_merge_amd", "csrc", f), "rb").read())
    if fields.get("source_sha256") != h.hexdigest():
        return None
    try:
        return float(fields[key])
    except (KeyError, ValueError):
        return None


def recorded_traffic(workload: str):
    """HBM bytes per ring launch from the committed counter summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{KERNEL}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        line = line.strip().strip("`")
        if "=" in line and " " not in line.split("=", 1)[0]:
            k, v = line.split("=", 1)
            fields[k] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def recorded_mfma_busy(workload: str):
    """Fraction of the ring launch's cycles with the matrix cores busy, from the committed counter
    summary (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x GRBM_GUI_ACTIVE per XCD), if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{KERNEL}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        line = line.strip().strip("`")
        if "=" in line and " " not in line.split("=", 1)[0]:
            k, v = line.split("=", 1)
            fields[k] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return float(fields["mfma_busy_frac"])
    except (KeyError, ValueError):
        return None


def backward(args, w, desc, q, k, v, src, sinks, out, lse, ws, stream, dense, eff_flops_chunk, fwd_step):
    """The --backward leg: ring_attn_bwd_1gpu steps, with the library recording HIP events around
    the ring backward's attention launches (the dq ring and the dk/dv launches) in every step."""
    dev = q.device
    fwd_step()
    dout = torch.from_numpy(np.random.default_rng(4242).standard_normal(tuple(q.shape), dtype=np.float32)).to(
        torch.bfloat16).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsinks = None if sinks is None else torch.empty(w.H, dtype=torch.float32, device=dev)
    del ws
    wsb = torch.empty(ram.ring_attn_bwd_workspace_bytes(desc, w.n_chunks, src), dtype=torch.uint8, device=dev)
    eff = BWD_FLOP_FACTOR * sum(eff_flops_chunk)

    def bstep():
        ram.ring_attn_bwd_1gpu(desc, w.n_chunks, w.q_shard, q, k, v, out, lse, dout, src, sinks, dq, dk, dv, dsinks,
                               wsb, stream=stream)

    for _ in range(args.warmup):
        bstep()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for a, b in evs:
        ram.set_kernel_events(a, b, stream=stream)
        bstep()
    e1.record(stream)
    ram.set_kernel_events()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tflops = eff / (ms * 1e-3) / 1e12
    log(f"backward step {ms:.3f} ms, {tflops:.1f} effective TFLOP/s ({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of peak)")
    kern = sorted(a.elapsed_time(b) for a, b in evs)
    kern_ms = float(np.median(kern))
    achieved = eff / (kern_ms * 1e-3) / 1e12
    ring_dq = w.dtype == "bf16" and w.n_chunks > 1
    launches = (1 if ring_dq else w.n_chunks) + w.n_chunks
    log(f"backward attention kernels median {kern_ms:.3f} ms per step (min {kern[0]:.3f}, max {kern[-1]:.3f}; "
        f"{launches} launches), {achieved:.1f} TFLOP/s")
    del wsb
    if args.copy_calibration:
        copy_calibration(dev)
    traffic = recorded_bwd(args.workload, "traffic", "traffic_bytes_per_step")   # HBM bytes per step
    traffic = None if traffic is None else int(traffic)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": ("attn_bwd_dq (one launch over all chunks) + attn_bwd_dkv (one launch per chunk)"
                           if ring_dq else "attn_bwd_dq + attn_bwd_dkv (one launch each per chunk)"),
                "launches_per_step": launches, "median_step_kernel_us": round(1e3 * kern_ms, 1),
                "timing": "HIP events around the ring backward's attention launches in each of the timed steps; "
                          "median",
                "flops_per_step": eff,
                "hbm_gbs": round(traffic / (kern_ms * 1e-3) / 1e9, 1) if traffic else None,
                "mfma_busy": recorded_bwd(args.workload, "counters", "mfma_busy_frac")}
    line = {
        "metric": METRIC_BWD, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "pass": "backward", "B": w.B, "H": w.H, "Hkv": w.Hkv, "Sq": w.Sq,
                   "Skv": w.Skv, "kv_chunks": w.n_chunks, "chunk": w.chunk, "D": w.D, "causal": w.causal,
                   "softcap": w.softcap, "sinks": w.sinks is not None, "q_shard": w.q_shard, "effective_flops": eff},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": None if args.no_cpu else cpu_baseline_bwd(w, min(args.cpu_rows, 256)),
    }
    print(json.dumps(line), flush=True)


def copy_calibration(dev):
    """A plain 256 MiB device copy, to scale the FETCH_SIZE / WRITE_SIZE counters."""
    a = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
    b2 = torch.empty_like(a)
    torch.cuda.synchronize()
    b2.copy_(a)                     # reads 256 MiB, writes 256 MiB
    torch.cuda.synchronize()
    del a, b2


def cpu_baseline_bwd(w, n_rows):
    """The float64 oracle backward over n_rows sampled query rows (all heads, all keys): the gradients of
    those rows' outputs, in the same 10*D FLOPs per allowed pair as the GPU's effective count."""
    import oracle
    from threadpoolctl import threadpool_info
    q, k, v, sinks = w.as_f64()
    qp, kp = w.positions()
    rows = wl.sampled_rows(w.Sq, w.chunk, n=n_rows, seed=2024)
    dout = np.random.default_rng(4243).standard_normal((w.B, n_rows, w.H, w.D))
    t0 = time.perf_counter()
    oracle.attention_bwd(q[:, rows], k, v, dout, scale=w.scale, q_pos=qp[:, rows], kv_pos=kp,
                         q_seg=None if w.q_seg is None else w.q_seg[:, rows], kv_seg=w.kv_seg, causal=w.causal,
                         softcap=w.softcap, sinks=sinks, dense=None if w.dense is None else w.dense[rows])
    dt = time.perf_counter() - t0
    pairs = 0
    for b in range(w.B):
        ok = oracle.allowed(qp[b, rows], kp[b], None if w.q_seg is None else w.q_seg[b, rows],
                            None if w.kv_seg is None else w.kv_seg[b], w.causal,
                            None if w.dense is None else w.dense[rows])
        pairs += int(ok.sum())
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    flops = 10.0 * w.D * w.H * pairs
    cores, model = host_cpu()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "cpu_model": model,
            "blas_threads": int(threads), "kind": "oracle",
            "sample": f"{n_rows} sampled of {w.Sq} query rows x all {w.H} heads x all {w.Skv} keys: float64 numpy "
                      f"oracle backward (its forward included), {dt:.2f} s",
            "sample_s": round(dt, 3), "extrapolated_full_s": round(dt * w.Sq / n_rows, 1),
            "extrapolation": "sample time x Sq / sampled rows (the oracle computes whole score rows, so its "
                             "time is linear in the rows); an estimate, not a measurement"}


def mask_builder_rate(w, desc, dense, bq, bk, dev, stream, reps):
    """The block-mask builder alone over the whole dense mask (one launch, all Sq x Skv pairs,
    at the kernel tile, bits stored), timed with HIP events on the stream it runs on.
    Algorithmic bytes: the mask bytes of every 32-key word the causal test does not clear
    (the builder reads no others), the bits of the PARTIAL tiles, and the classes and lists."""
    d = ram.Desc(**{**desc.__dict__, "Skv": w.Skv, "block_q": bq, "block_kv": bk})
    src = ram.MaskSrc(q_pos_base=w.q_shard * w.Sq if w.q_shard >= 0 else 0, dense=dense)
    bm = ram.alloc_block_mask(d, device=dev, with_bits=True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ram.build_block_mask(d, src, bm, stream=stream)
    a.record(stream)
    for _ in range(reps):
        ram.build_block_mask(d, src, bm, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * a.elapsed_time(b) / reps
    q0 = src.q_pos_base
    rows = np.arange(w.Sq, dtype=np.int64) + q0
    read = int(np.minimum(w.Skv, ((rows + 1 + 31) // 32) * 32).clip(min=0).sum()) if w.causal else w.Sq * w.Skv
    n_tiles = bm.nQb * bm.nKb
    n_partial = int((bm.tile_class[:n_tiles] == ram.RAM_TILE_PARTIAL).sum().item())
    nbytes = read + n_partial * bm.tile_words * 4 + n_tiles * 5 + bm.nQb * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"mask builder over [{w.Sq}, {w.Skv}]: {us:.1f} us, {gbs:.0f} GB/s of {nbytes / 1e6:.1f} MB")
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "kernel": "block_mask_kernel", "launch_us": round(us, 1),
            "bytes_per_launch": nbytes, "partial_tiles": n_partial, "tiles": n_tiles}


def cpu_baseline(w, n_rows: int):
    import oracle
    from threadpoolctl import threadpool_info
    rows = wl.sampled_rows(w.Sq, w.chunk, n=n_rows, seed=2024)
    q, k, v, sinks = w.as_f64()
    qp, kp = w.positions()
    t0 = time.perf_counter()
    oracle.attention(q, k, v, scale=w.scale, q_pos=qp, kv_pos=kp, q_seg=w.q_seg, kv_seg=w.kv_seg,
                     causal=w.causal, softcap=w.softcap, sinks=sinks, dense=w.dense, rows=rows)
    dt = time.perf_counter() - t0
    pairs = 0
    for b in range(w.B):
        ok = oracle.allowed(qp[b, rows], kp[b], None if w.q_seg is None else w.q_seg[b, rows],
                            None if w.kv_seg is None else w.kv_seg[b], w.causal,
                            None if w.dense is None else w.dense[rows])
        pairs += int(ok.sum())
    flops = 4.0 * w.D * w.H * pairs
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    cores, model = host_cpu()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "cpu_model": model,
            "blas_threads": int(threads), "kind": "oracle",
            "sample": f"{len(rows)} of {w.Sq} query rows x all {w.H} heads x all {w.Skv} keys, float64 "
                      f"numpy oracle (full score rows, BLAS dgemm), {dt:.2f} s",
            "sample_s": round(dt, 3), "extrapolated_full_s": round(dt * w.Sq / len(rows), 1),
            "extrapolation": "sample time x Sq / sampled rows (the oracle computes whole score rows, so its "
                             "time is linear in the rows); an estimate, not a measurement"}


def mfma_rates(dev, stream) -> dict:
    """The dense bf16 MFMA rate this GPU sustains from registers (ram_mfma_probe), with all-zero and
    with pseudo-random operands: the clock of the matrix cores follows the operands' switching activity,
    so the published peak is reached only with the former."""
    n_blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(n_blocks * 512, dtype=torch.float32, device=dev)
    iters = 2000
    flops = 32768.0 * 32 * iters * 8 * n_blocks       # 32 MFMAs per wave and iteration, 8 waves per block
    res = {}
    for name, kind in (("zeros", 0), ("random", 1)):
        ram.mfma_probe(n_blocks, 50, kind, out, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ram.mfma_probe(n_blocks, iters, kind, out, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = round(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    res["unit"] = "TFLOP/s"
    res["probe"] = f"ram_mfma_probe, {n_blocks} workgroups x 8 waves, 32x32x16 bf16 MFMAs from registers"
    return res


def graph_leg(args, step, eff_flops, out, lse):
    """The same step captured once in a HIP graph and replayed: the ring call launches only
    kernels on its stream (no allocation, memset or host synchronisation), so the replays run the
    identical work without the host's launch gaps between the kernels. The first replay's result
    is checked bit for bit against the eager step's."""
    ref_out, ref_lse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        step(torch.cuda.current_stream())
    out.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(out, ref_out) and torch.equal(lse, ref_lse))
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tflops = eff_flops / (ms * 1e-3) / 1e12
    log(f"graph replay: step {ms:.3f} ms, {tflops:.1f} effective TFLOP/s; replay equals the eager step: {same}")
    return {"ms_per_step": round(ms, 4), "value": round(tflops, 2), "replay_equals_eager": same,
            "timing": "K replays of the captured step between two events"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c5", choices=["c5", "c4", "c4mqa", "c3", "c2", "c5dense"])
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--backward", action="store_true", help="time the ring backward instead of the forward")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed (no host launch gaps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (to scale FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); this path has no multi-GPU "
              "mode: the ring's chunks run as a sequential loop on one device.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda"
    torch.cuda.set_device(0)

    log(f"generating workload {args.workload} ...")
    w = workload(args.workload)
    dcode = ram.RAM_BF16 if w.dtype == "bf16" else ram.RAM_F32
    desc = ram.Desc(B=w.B, Sq=w.Sq, Skv=w.chunk, H=w.H, Hkv=w.Hkv, D=w.D, dtype=dcode, scale=w.scale,
                    softcap=w.softcap or 0.0, causal=w.causal)
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    sinks = None if w.sinks is None else w.sinks.to(dev)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    dense = dense_tensor(w, dev)
    src = ram.MaskSrc(q_pos=t(w.q_pos), kv_pos=t(w.kv_pos), q_seg=t(w.q_seg), kv_seg=t(w.kv_seg),
                      dense=dense, dense_chunk_step=w.chunk if dense is not None else 0)
    out = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.Sq, dtype=torch.float32, device=dev)
    ws = torch.empty(ram.ring_attn_workspace_bytes(desc, w.n_chunks, src), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    ref_tiles = independent_tiles(w)
    lib_tiles = tile_counts(w, desc, dev, REF_TILE, REF_TILE, dense)
    eff_flops_chunk = [4.0 * w.D * w.H * n * REF_TILE * REF_TILE for n in ref_tiles]
    eff_flops = sum(eff_flops_chunk)
    log(f"non-empty {REF_TILE}x{REF_TILE} tiles per chunk: {ref_tiles} (library: "
        f"{'agrees' if lib_tiles == ref_tiles else lib_tiles}); effective FLOPs {eff_flops:.4e}")
    tiles_info = {"nonempty_tiles_128": sum(ref_tiles), "library_count_agrees": lib_tiles == ref_tiles}

    def step(on=None):
        ram.ring_attn_fwd_1gpu(desc, w.n_chunks, w.q_shard, q, k, v, src, sinks, out, lse, ws,
                               stream=stream if on is None else on)

    if args.backward:
        return backward(args, w, desc, q, k, v, src, sinks, out, lse, ws, stream, dense, eff_flops_chunk, step)

    bq, bk = ram.kernel_tile(dcode, w.D)
    alt = dcode == ram.RAM_BF16 and w.D == 128    # one attention launch per step; else one per chunk
    launches = 1 if alt else w.n_chunks
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed window: every step also has the library record HIP events on its stream right
    # around the attention launch(es), so the kernel's time comes from the same steps.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for a, b in evs:
        ram.set_kernel_events(a, b, stream=stream)
        step()
    e1.record(stream)
    ram.set_kernel_events()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tflops = eff_flops / (ms * 1e-3) / 1e12
    log(f"step {ms:.3f} ms, {tflops:.1f} effective TFLOP/s ({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of peak)")
    kern = sorted(a.elapsed_time(b) for a, b in evs)
    kern_ms = float(np.median(kern))
    if kern_ms > ms:
        log(f"warning: median kernel time {kern_ms:.3f} ms above the mean step time {ms:.3f} ms")
    achieved = eff_flops / (kern_ms * 1e-3) / 1e12
    log(f"attention kernel median {kern_ms:.3f} ms per step (min {kern[0]:.3f}, max {kern[-1]:.3f}; "
        f"{launches} launch(es)), {achieved:.1f} TFLOP/s")
    split = alt and ring_splits(w, bq)
    bits = any(x is not None for x in (dense, w.kv_pos, w.q_seg, w.kv_seg))   # masked from stored bits
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic(args.workload) if alt else None,
                "kernel": ring_kernel_name(w.softcap, bits, split, ring_packs_v(w)) if alt else "per-chunk launches",
                "launches_per_step": launches, "median_step_kernel_us": round(1e3 * kern_ms, 1),
                "mean_launch_us": round(1e3 * kern_ms / launches, 2),
                "timing": "HIP events around the attention launch in each of the timed steps; median",
                "flops_per_launch_mean": eff_flops / launches}
    graph = graph_leg(args, step, eff_flops, out, lse) if args.graph else None
    measured = mfma_rates(dev, stream)
    roofline["measured_peak_random"] = measured["random"]
    roofline["frac_of_measured_random"] = round(achieved / measured["random"], 4)
    # rocprofv3 counters of the same launch, recorded in profiles/ (null once the kernel changed)
    roofline["mfma_busy"] = recorded_mfma_busy(args.workload) if alt else None
    roofline["hbm_gbs"] = (round(roofline["traffic"] / (kern_ms * 1e-3 / launches) / 1e9, 1)
                           if roofline["traffic"] else None)
    log(f"MFMA probe: {measured['zeros']} TFLOP/s with zero operands, {measured['random']} with random ones")
    builder = None if dense is None else mask_builder_rate(w, desc, dense, bq, bk, dev, stream,
                                                            max(1, args.steps // 2))
    if args.copy_calibration:
        copy_calibration(dev)

    cpu = None
    if not args.no_cpu:
        log(f"timing the float64 oracle on {args.cpu_rows} sampled rows ...")
        cpu = cpu_baseline(w, args.cpu_rows)
        log(f"oracle: {cpu['value'] * 1e3:.3f} GFLOP/s ({cpu['cores']} cores, {cpu['blas_threads']} BLAS "
            f"threads, {cpu['cpu_model']}); full size extrapolated {cpu['extrapolated_full_s']} s")

    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "Sq": w.Sq, "Skv": w.Skv,
                   "kv_chunks": w.n_chunks, "chunk": w.chunk, "D": w.D, "causal": w.causal,
                   "softcap": w.softcap, "sinks": w.sinks is not None, "q_shard": w.q_shard,
                   "effective_flops": eff_flops, **tiles_info},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "mfma_measured": measured,
    }
    if builder is not None:
        line["mask_builder"] = builder
    if graph is not None:
        line["graph"] = graph
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
