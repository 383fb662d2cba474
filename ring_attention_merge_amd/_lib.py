"""ctypes binding of libram (include/ram.h): argument marshalling only.

Every step of the path runs in the HIP library; this module turns torch
tensors into device pointers and the current HIP stream, checks that each
tensor is on the GPU with the dtype and size the call reads (so a wrong tensor
can never reach a kernel), and raises ``RamError`` with the library's message
on a non-OK status. It fails loudly when libram.so is missing: there is no
CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libram.so")

RAM_OK, RAM_ERR_INVALID, RAM_ERR_UNSUPPORTED, RAM_ERR_WORKSPACE, RAM_ERR_HIP = range(5)
RAM_F32, RAM_BF16 = 0, 1
RAM_TILE_EMPTY, RAM_TILE_PARTIAL, RAM_TILE_FULL = 0, 1, 2
RAM_OUT_WRITE, RAM_OUT_MERGE = 0, 1
RAM_PAD_SEGMENT_ID = -1

EXPORTS = ("build_block_mask", "attn_fwd_chunk", "lse_merge", "ring_attn_fwd_1gpu",
           "ring_attn_workspace_bytes", "ram_kernel_tile", "ram_bwd_kernel_tile", "ram_last_error", "attn_bwd_prep",
           "attn_bwd_chunk", "ring_attn_bwd_1gpu", "ring_attn_bwd_workspace_bytes", "ring_attn_fwd_masks",
           "ring_attn_bwd_masks", "ring_attn_fwd_1gpu_noalloc", "ram_mfma_probe", "ram_set_kernel_events")


class RamError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libram status {status}: {message}")
        self.status = status


class c_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Sq", ctypes.c_int32), ("Skv", ctypes.c_int32),
                ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("q_stride_b", ctypes.c_int64),
                ("kv_stride_b", ctypes.c_int64), ("scale", ctypes.c_float),
                ("softcap", ctypes.c_float), ("causal", ctypes.c_int32),
                ("block_q", ctypes.c_int32), ("block_kv", ctypes.c_int32)]


class c_ring_masks(ctypes.Structure):
    _fields_ = [("cls_off", ctypes.c_int64), ("cnt_off", ctypes.c_int64), ("col_off", ctypes.c_int64),
                ("bits_off", ctypes.c_int64), ("order_off", ctypes.c_int64), ("block_q", ctypes.c_int32),
                ("block_kv", ctypes.c_int32),
                ("nQb", ctypes.c_int32), ("nKb", ctypes.c_int32), ("tile_words", ctypes.c_int32)]


class c_mask_src(ctypes.Structure):
    _fields_ = [("q_pos", ctypes.c_void_p), ("kv_pos", ctypes.c_void_p),
                ("q_pos_base", ctypes.c_int32), ("kv_pos_base", ctypes.c_int32),
                ("q_seg", ctypes.c_void_p), ("kv_seg", ctypes.c_void_p),
                ("q_meta_stride_b", ctypes.c_int64), ("kv_meta_stride_b", ctypes.c_int64),
                ("dense", ctypes.c_void_p), ("dense_ld", ctypes.c_int64),
                ("dense_chunk_step", ctypes.c_int64)]


class c_block_mask(ctypes.Structure):
    _fields_ = [("tile_class", ctypes.c_void_p), ("row_cnt", ctypes.c_void_p),
                ("col_idx", ctypes.c_void_p), ("bits", ctypes.c_void_p),
                ("col_cnt", ctypes.c_void_p), ("row_idx", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libram.so (once). Raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libram.so not found at {path}; build it with "
                          "`python -m ring_attention_merge_amd.build` (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, i32, f32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
    P = ctypes.POINTER
    lib.build_block_mask.argtypes = [P(c_desc), P(c_mask_src), P(c_block_mask), vp]
    lib.attn_fwd_chunk.argtypes = [P(c_desc), vp, vp, vp, P(c_mask_src), P(c_block_mask), f32p, i32,
                                   f32p, f32p, vp]
    lib.lse_merge.argtypes = [i32, i32, i32, i32, f32p, f32p, f32p, f32p, vp]
    lib.ring_attn_fwd_1gpu.argtypes = [P(c_desc), i32, i32, vp, vp, vp, P(c_mask_src), f32p, vp, f32p,
                                       vp, ctypes.c_size_t, vp]
    lib.ring_attn_workspace_bytes.argtypes = [P(c_desc), i32, P(c_mask_src)]
    lib.ring_attn_fwd_1gpu_noalloc.argtypes = [P(c_desc), i32, i32, vp, vp, vp, P(c_mask_src), f32p, vp, f32p, vp]
    lib.ring_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.ram_kernel_tile.argtypes = [i32, i32, P(i32), P(i32)]
    lib.ram_bwd_kernel_tile.argtypes = [i32, i32, P(i32), P(i32)]
    lib.attn_bwd_prep.argtypes = [P(c_desc), vp, vp, f32p, f32p, f32p, f32p, vp]
    lib.attn_bwd_chunk.argtypes = [P(c_desc), vp, vp, vp, vp, f32p, f32p, P(c_mask_src), P(c_block_mask), i32,
                                   f32p, f32p, f32p, vp]
    lib.ring_attn_bwd_1gpu.argtypes = [P(c_desc), i32, i32, vp, vp, vp, vp, f32p, vp, P(c_mask_src), f32p, vp,
                                       vp, vp, f32p, vp, ctypes.c_size_t, vp]
    lib.ring_attn_bwd_workspace_bytes.argtypes = [P(c_desc), i32, P(c_mask_src)]
    lib.ring_attn_fwd_masks.argtypes = [P(c_desc), i32, P(c_mask_src), P(c_ring_masks)]
    lib.ring_attn_bwd_masks.argtypes = [P(c_desc), i32, P(c_mask_src), P(c_ring_masks)]
    lib.ring_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ram_last_error.argtypes = []
    lib.ram_last_error.restype = ctypes.c_char_p
    lib.ram_mfma_probe.argtypes = [i32, i32, i32, f32p, vp]
    lib.ram_set_kernel_events.argtypes = [vp, vp]
    for name in ("build_block_mask", "attn_fwd_chunk", "lse_merge", "ring_attn_fwd_1gpu", "ram_kernel_tile",
                 "ram_bwd_kernel_tile",
                 "attn_bwd_prep", "attn_bwd_chunk", "ring_attn_bwd_1gpu", "ram_mfma_probe",
                 "ram_set_kernel_events", "ring_attn_fwd_masks", "ring_attn_bwd_masks", "ring_attn_fwd_1gpu_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != RAM_OK:
        raise RamError(status, load().ram_last_error().decode())


# ------------------------------------------------------------------------------ descriptors
@dataclass
class Desc:
    """Python side of ram_attn_desc (sizes, dtype, scale, soft cap, causal, tile)."""
    B: int
    Sq: int
    Skv: int
    H: int
    Hkv: int
    D: int
    dtype: int = RAM_BF16
    scale: float = 1.0
    softcap: float = 0.0
    causal: bool = True
    block_q: int = 128
    block_kv: int = 64
    q_stride_b: int = 0
    kv_stride_b: int = 0

    def c(self) -> c_desc:
        return c_desc(self.B, self.Sq, self.Skv, self.H, self.Hkv, self.D, self.dtype, self.q_stride_b,
                      self.kv_stride_b, self.scale, self.softcap if self.softcap else 0.0,
                      int(self.causal), self.block_q, self.block_kv)


@dataclass
class MaskSrc:
    """Python side of ram_mask_src: int32 CUDA tensors or None (sequential / no segments),
    and an optional dense uint8 [Sq, dense_ld] mask (nonzero = allowed)."""
    q_pos: Optional[torch.Tensor] = None
    kv_pos: Optional[torch.Tensor] = None
    q_pos_base: int = 0
    kv_pos_base: int = 0
    q_seg: Optional[torch.Tensor] = None
    kv_seg: Optional[torch.Tensor] = None
    q_meta_stride_b: int = 0
    kv_meta_stride_b: int = 0
    dense: Optional[torch.Tensor] = None
    dense_ld: int = 0
    dense_chunk_step: int = 0

    def c(self, B: int, Sq: int, kv_len: int, dense_cols: Optional[int] = None) -> c_mask_src:
        for name, t, S, st in (("q_pos", self.q_pos, Sq, self.q_meta_stride_b),
                               ("q_seg", self.q_seg, Sq, self.q_meta_stride_b),
                               ("kv_pos", self.kv_pos, kv_len, self.kv_meta_stride_b),
                               ("kv_seg", self.kv_seg, kv_len, self.kv_meta_stride_b)):
            if t is not None:
                _need(t, name, torch.int32, (B - 1) * (st or S) + S if B > 0 else 0)
        if self.dense is not None:
            cols = kv_len if dense_cols is None else dense_cols
            ld = self.dense_ld or cols
            _need(self.dense, "dense", torch.uint8, (Sq - 1) * ld + cols if Sq > 0 and ld >= cols else 0)
        return c_mask_src(_ptr(self.q_pos), _ptr(self.kv_pos), self.q_pos_base, self.kv_pos_base,
                          _ptr(self.q_seg), _ptr(self.kv_seg), self.q_meta_stride_b, self.kv_meta_stride_b,
                          _ptr(self.dense), self.dense_ld, self.dense_chunk_step)


@dataclass
class BlockMask:
    """Python side of ram_block_mask: uint8 / int32 CUDA tensors, plus the optional
    int32 tile bits (uint32 words in the C ABI) of PARTIAL tiles."""
    tile_class: torch.Tensor
    row_cnt: torch.Tensor
    col_idx: torch.Tensor
    nQb: int = 0
    nKb: int = 0
    bits: Optional[torch.Tensor] = None
    tile_words: int = 0   # block_q * ceil(block_kv / 32)
    col_cnt: Optional[torch.Tensor] = None
    row_idx: Optional[torch.Tensor] = None

    def c(self, B: int) -> c_block_mask:
        _need(self.tile_class, "tile_class", torch.uint8, B * self.nQb * self.nKb)
        _need(self.row_cnt, "row_cnt", torch.int32, B * self.nQb)
        _need(self.col_idx, "col_idx", torch.int32, B * self.nQb * self.nKb)
        if self.bits is not None:
            _need(self.bits, "bits", torch.int32, B * self.nQb * self.nKb * self.tile_words)
        if self.col_cnt is not None:
            _need(self.col_cnt, "col_cnt", torch.int32, B * self.nKb)
            _need(self.row_idx, "row_idx", torch.int32, B * self.nKb * self.nQb)
        return c_block_mask(_ptr(self.tile_class), _ptr(self.row_cnt), _ptr(self.col_idx), _ptr(self.bits),
                            _ptr(self.col_cnt), _ptr(self.row_idx))


def alloc_block_mask(desc: Desc, device="cuda", with_bits: bool = False, with_cols: bool = False) -> BlockMask:
    """Allocate the block-mask arrays for desc's shape and tile (and the tile bits, and the
    transposed lists the backward walks)."""
    nQb = -(-desc.Sq // desc.block_q)
    nKb = -(-desc.Skv // desc.block_kv)
    n = max(1, desc.B * nQb * nKb)
    tw = desc.block_q * (-(-desc.block_kv // 32))
    bits = torch.zeros(n * tw, dtype=torch.int32, device=device) if with_bits else None
    cc = torch.empty(max(1, desc.B * nKb), dtype=torch.int32, device=device) if with_cols else None
    ri = torch.empty(n, dtype=torch.int32, device=device) if with_cols else None
    return BlockMask(torch.empty(n, dtype=torch.uint8, device=device),
                     torch.empty(max(1, desc.B * nQb), dtype=torch.int32, device=device),
                     torch.empty(n, dtype=torch.int32, device=device), nQb, nKb, bits, tw, cc, ri)


# ------------------------------------------------------------------------------ helpers
def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, numel: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (device {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, the call reads {numel}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _tdtype(dtype: int):
    return torch.bfloat16 if dtype == RAM_BF16 else torch.float32


def _span(B, stride, dense):
    return 0 if B == 0 else (B - 1) * (stride or dense) + dense


# ------------------------------------------------------------------------------ entry points
def kernel_tile(dtype: int, D: int):
    """ram_kernel_tile: the (block_q, block_kv) mask tile attn_fwd_chunk needs."""
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    _check(load().ram_kernel_tile(dtype, D, ctypes.byref(bq), ctypes.byref(bk)))
    return bq.value, bk.value


def bwd_kernel_tile(dtype: int, D: int):
    """ram_bwd_kernel_tile: the (block_q, block_kv) mask tile attn_bwd_chunk needs."""
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    _check(load().ram_bwd_kernel_tile(dtype, D, ctypes.byref(bq), ctypes.byref(bk)))
    return bq.value, bk.value


def build_block_mask(desc: Desc, src: MaskSrc, out: BlockMask, stream=None):
    """build_block_mask: tile classes and compacted non-empty tile lists."""
    cd, cs = desc.c(), src.c(desc.B, desc.Sq, desc.Skv)
    cb = out.c(desc.B)
    _check(load().build_block_mask(ctypes.byref(cd), ctypes.byref(cs), ctypes.byref(cb), _stream(stream)))


def attn_fwd_chunk(desc: Desc, q, k, v, src: MaskSrc, mask: BlockMask, sinks, mode: int, out, lse,
                   stream=None):
    """attn_fwd_chunk: one KV chunk, written (mode 0) or merged (mode 1) into out / lse."""
    dt = _tdtype(desc.dtype)
    _need(q, "q", dt, _span(desc.B, desc.q_stride_b, desc.Sq * desc.H * desc.D))
    if desc.Skv > 0:
        _need(k, "k", dt, _span(desc.B, desc.kv_stride_b, desc.Skv * desc.Hkv * desc.D))
        _need(v, "v", dt, _span(desc.B, desc.kv_stride_b, desc.Skv * desc.Hkv * desc.D))
    _need(out, "out", torch.float32, desc.B * desc.Sq * desc.H * desc.D)
    _need(lse, "lse", torch.float32, desc.B * desc.H * desc.Sq)
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, desc.H)
    cd, cs, cb = desc.c(), src.c(desc.B, desc.Sq, desc.Skv), mask.c(desc.B)
    _check(load().attn_fwd_chunk(ctypes.byref(cd), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs),
                                 ctypes.byref(cb), _ptr(sinks), mode, _ptr(out), _ptr(lse),
                                 _stream(stream)))


def set_kernel_events(start=None, stop=None, stream=None):
    """ram_set_kernel_events: torch.cuda.Event pair (enable_timing) that this thread's ring forward
    and backward calls record around their attention launches; no arguments to stop. Both events are recorded
    once here on `stream` (torch measures only events it has seen recorded); the ring calls record
    them again at their launches, and elapsed_time reads those last records."""
    if (start is None) != (stop is None):
        raise ValueError("set both events or neither")
    if start is not None:
        st = torch.cuda.current_stream() if stream is None else stream
        start.record(st)
        stop.record(st)
    h = lambda e: None if e is None else e.cuda_event
    _check(load().ram_set_kernel_events(h(start), h(stop)))


def mfma_probe(n_blocks: int, iters: int, operands: int, out, stream=None):
    """ram_mfma_probe: n_blocks x 8 waves of register-fed bf16 MFMAs (operands 0: zeros, 1: random);
    out float32 [n_blocks * 512] receives a checksum per thread."""
    _need(out, "out", torch.float32, n_blocks * 512)
    st = load().ram_mfma_probe(n_blocks, iters, operands, _ptr(out), _stream(stream))
    if st != RAM_OK:
        raise RamError(st, f"ram_mfma_probe(n_blocks={n_blocks}, iters={iters}, operands={operands})")


def lse_merge(out_acc, lse_acc, out_blk, lse_blk, stream=None):
    """lse_merge: fold (out_blk, lse_blk) into (out_acc, lse_acc) in place; out [B,Sq,H,D]."""
    B, Sq, H, D = out_acc.shape
    n = B * Sq * H * D
    for name, t, m in (("out_acc", out_acc, n), ("out_blk", out_blk, n), ("lse_acc", lse_acc, B * H * Sq),
                       ("lse_blk", lse_blk, B * H * Sq)):
        _need(t, name, torch.float32, m)
    _check(load().lse_merge(B, Sq, H, D, _ptr(out_acc), _ptr(lse_acc), _ptr(out_blk), _ptr(lse_blk),
                            _stream(stream)))


def ring_attn_workspace_bytes(desc: Desc, n_chunks: int, src: Optional[MaskSrc] = None) -> int:
    cd = desc.c()
    if src is None:
        return int(load().ring_attn_workspace_bytes(ctypes.byref(cd), n_chunks, None))
    # only which arrays are given matters for the size (they may live anywhere)
    cs = c_mask_src(_ptr(src.q_pos), _ptr(src.kv_pos), 0, 0, _ptr(src.q_seg), _ptr(src.kv_seg), 0, 0,
                    _ptr(src.dense), src.dense_ld, src.dense_chunk_step)
    return int(load().ring_attn_workspace_bytes(ctypes.byref(cd), n_chunks, ctypes.byref(cs)))


def ring_attn_fwd_1gpu(desc: Desc, n_chunks: int, q_shard: int, q, k_all, v_all, src: MaskSrc, sinks,
                       out, lse, workspace, stream=None):
    """ring_attn_fwd_1gpu: all KV chunks in (ring) order, merged by LSE, cast to the q dtype."""
    dt = _tdtype(desc.dtype)
    kv_len = n_chunks * desc.Skv
    _need(q, "q", dt, _span(desc.B, desc.q_stride_b, desc.Sq * desc.H * desc.D))
    if kv_len > 0:
        _need(k_all, "k_all", dt, _span(desc.B, desc.kv_stride_b, kv_len * desc.Hkv * desc.D))
        _need(v_all, "v_all", dt, _span(desc.B, desc.kv_stride_b, kv_len * desc.Hkv * desc.D))
    _need(out, "out", dt, desc.B * desc.Sq * desc.H * desc.D)
    _need(lse, "lse", torch.float32, desc.B * desc.H * desc.Sq)
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, desc.H)
    _need(workspace, "workspace", torch.uint8, 0)
    dense_cols = desc.Skv + (n_chunks - 1) * src.dense_chunk_step
    cd, cs = desc.c(), src.c(desc.B, desc.Sq, kv_len, dense_cols)
    _check(load().ring_attn_fwd_1gpu(ctypes.byref(cd), n_chunks, q_shard, _ptr(q), _ptr(k_all), _ptr(v_all),
                                     ctypes.byref(cs), _ptr(sinks), _ptr(out), _ptr(lse), _ptr(workspace),
                                     workspace.numel(), _stream(stream)))


def ring_attn_fwd_1gpu_noalloc(desc: Desc, n_chunks: int, q_shard: int, q, k_all, v_all, src: MaskSrc, sinks,
                               out, lse, stream=None):
    """ring_attn_fwd_1gpu_noalloc: ring_attn_fwd_1gpu with the library's static per-GPU scratch
    instead of a workspace (no device allocation; calls that overlap on one GPU race)."""
    dt = _tdtype(desc.dtype)
    kv_len = n_chunks * desc.Skv
    _need(q, "q", dt, _span(desc.B, desc.q_stride_b, desc.Sq * desc.H * desc.D))
    if kv_len > 0:
        _need(k_all, "k_all", dt, _span(desc.B, desc.kv_stride_b, kv_len * desc.Hkv * desc.D))
        _need(v_all, "v_all", dt, _span(desc.B, desc.kv_stride_b, kv_len * desc.Hkv * desc.D))
    _need(out, "out", dt, desc.B * desc.Sq * desc.H * desc.D)
    _need(lse, "lse", torch.float32, desc.B * desc.H * desc.Sq)
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, desc.H)
    dense_cols = desc.Skv + (n_chunks - 1) * src.dense_chunk_step
    cd, cs = desc.c(), src.c(desc.B, desc.Sq, kv_len, dense_cols)
    _check(load().ring_attn_fwd_1gpu_noalloc(ctypes.byref(cd), n_chunks, q_shard, _ptr(q), _ptr(k_all), _ptr(v_all),
                                             ctypes.byref(cs), _ptr(sinks), _ptr(out), _ptr(lse), _stream(stream)))


# ------------------------------------------------------------------------------ backward
def attn_bwd_prep(desc: Desc, out, dout, lse, sinks, delta, dsinks, stream=None):
    """attn_bwd_prep: delta [2,B,H,Sq] (rowsum(dout * out), then the base-2 lse) and, with sinks, dsinks [H]."""
    dt = _tdtype(desc.dtype)
    n = desc.B * desc.Sq * desc.H * desc.D
    _need(out, "out", dt, n)
    _need(dout, "dout", dt, n)
    _need(lse, "lse", torch.float32, desc.B * desc.H * desc.Sq)
    _need(delta, "delta", torch.float32, 2 * desc.B * desc.H * desc.Sq)
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, desc.H)
        _need(dsinks, "dsinks", torch.float32, desc.H)
    cd = desc.c()
    _check(load().attn_bwd_prep(ctypes.byref(cd), _ptr(out), _ptr(dout), _ptr(lse), _ptr(sinks), _ptr(delta),
                                _ptr(dsinks), _stream(stream)))


def attn_bwd_chunk(desc: Desc, q, k, v, dout, lse, delta, src: MaskSrc, mask: BlockMask, dq_mode: int, dq, dk, dv,
                   stream=None):
    """attn_bwd_chunk: float32 dq written (mode 0) or added (mode 1); float32 dk, dv written."""
    dt = _tdtype(desc.dtype)
    _need(q, "q", dt, _span(desc.B, desc.q_stride_b, desc.Sq * desc.H * desc.D))
    _need(dout, "dout", dt, desc.B * desc.Sq * desc.H * desc.D)
    _need(lse, "lse", torch.float32, desc.B * desc.H * desc.Sq)
    _need(delta, "delta", torch.float32, 2 * desc.B * desc.H * desc.Sq)
    _need(dq, "dq", torch.float32, desc.B * desc.Sq * desc.H * desc.D)
    kvn = _span(desc.B, desc.kv_stride_b, desc.Skv * desc.Hkv * desc.D)
    if desc.Skv > 0:
        for name, t, tt in (("k", k, dt), ("v", v, dt), ("dk", dk, torch.float32), ("dv", dv, torch.float32)):
            _need(t, name, tt, kvn)
    cd, cs, cb = desc.c(), src.c(desc.B, desc.Sq, desc.Skv), mask.c(desc.B)
    _check(load().attn_bwd_chunk(ctypes.byref(cd), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
                                 ctypes.byref(cs), ctypes.byref(cb), dq_mode, _ptr(dq), _ptr(dk), _ptr(dv),
                                 _stream(stream)))


def ring_attn_bwd_workspace_bytes(desc: Desc, n_chunks: int, src: Optional[MaskSrc] = None) -> int:
    cd = desc.c()
    if src is None:
        return int(load().ring_attn_bwd_workspace_bytes(ctypes.byref(cd), n_chunks, None))
    cs = c_mask_src(0, 0, 0, 0, 0, 0, 0, 0, _ptr(src.dense), src.dense_ld, src.dense_chunk_step)
    return int(load().ring_attn_bwd_workspace_bytes(ctypes.byref(cd), n_chunks, ctypes.byref(cs)))


def _ring_masks(fn, desc: Desc, n_chunks: int, src: Optional[MaskSrc]) -> dict:
    cd = desc.c()
    cs = None if src is None else c_mask_src(_ptr(src.q_pos), _ptr(src.kv_pos), 0, 0, _ptr(src.q_seg),
                                            _ptr(src.kv_seg), 0, 0, _ptr(src.dense), src.dense_ld,
                                            src.dense_chunk_step)
    m = c_ring_masks()
    _check(fn(ctypes.byref(cd), n_chunks, None if cs is None else ctypes.byref(cs), ctypes.byref(m)))
    return {f: getattr(m, f) for f, _ in c_ring_masks._fields_}


def ring_attn_fwd_masks(desc: Desc, n_chunks: int, src: Optional[MaskSrc] = None) -> dict:
    """ring_attn_fwd_masks: where ring_attn_fwd_1gpu's workspace holds each chunk's block mask
    (byte offsets cls_off, cnt_off, col_off, bits_off (-1: none), and order_off, the rows' order
    (-1: none); block_q, block_kv, nQb, nKb, tile_words)."""
    return _ring_masks(load().ring_attn_fwd_masks, desc, n_chunks, src)


def ring_attn_bwd_masks(desc: Desc, n_chunks: int, src: Optional[MaskSrc] = None) -> dict:
    """ring_attn_bwd_masks: the same for ring_attn_bwd_1gpu's workspace."""
    return _ring_masks(load().ring_attn_bwd_masks, desc, n_chunks, src)


def ring_attn_bwd_1gpu(desc: Desc, n_chunks: int, q_shard: int, q, k_all, v_all, out, lse, dout, src: MaskSrc,
                       sinks, dq, dk_all, dv_all, dsinks, workspace, stream=None):
    """ring_attn_bwd_1gpu: gradients of ring_attn_fwd_1gpu (dq, dk_all, dv_all in the q dtype; dsinks float32)."""
    dt = _tdtype(desc.dtype)
    kv_len = n_chunks * desc.Skv
    n = desc.B * desc.Sq * desc.H * desc.D
    _need(q, "q", dt, _span(desc.B, desc.q_stride_b, desc.Sq * desc.H * desc.D))
    for name, t in (("out", out), ("dout", dout), ("dq", dq)):
        _need(t, name, dt, n)
    _need(lse, "lse", torch.float32, desc.B * desc.H * desc.Sq)
    if kv_len > 0:
        kvn = _span(desc.B, desc.kv_stride_b, kv_len * desc.Hkv * desc.D)
        for name, t in (("k_all", k_all), ("v_all", v_all), ("dk_all", dk_all), ("dv_all", dv_all)):
            _need(t, name, dt, kvn)
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, desc.H)
        _need(dsinks, "dsinks", torch.float32, desc.H)
    _need(workspace, "workspace", torch.uint8, 0)
    dense_cols = desc.Skv + (n_chunks - 1) * src.dense_chunk_step
    cd, cs = desc.c(), src.c(desc.B, desc.Sq, kv_len, dense_cols)
    _check(load().ring_attn_bwd_1gpu(ctypes.byref(cd), n_chunks, q_shard, _ptr(q), _ptr(k_all), _ptr(v_all),
                                     _ptr(out), _ptr(lse), _ptr(dout), ctypes.byref(cs), _ptr(sinks), _ptr(dq),
                                     _ptr(dk_all), _ptr(dv_all), _ptr(dsinks), _ptr(workspace), workspace.numel(),
                                     _stream(stream)))
