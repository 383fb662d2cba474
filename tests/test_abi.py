"""C ABI checks that need no GPU: exported symbols and host-side argument validation.

Every call here fails validation (or is an empty no-op) before anything is
enqueued, so no device is touched; the pointers are fake but aligned and are
never dereferenced on these paths.
"""
import ctypes
import os
import re

import pytest
import torch

import ring_attention_merge_amd as ram
from ring_attention_merge_amd import _lib, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000            # 16-byte (and 256-byte) aligned, never dereferenced
FAKE2 = 0x200000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    return ram.load()


def _header_functions():
    src = open(os.path.join(ROOT, "include", "ram.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_every_header_symbol_is_exported(lib):
    names = _header_functions()
    assert set(names) == {"build_block_mask", "attn_fwd_chunk", "lse_merge", "ring_attn_fwd_1gpu",
                          "ring_attn_workspace_bytes", "ram_kernel_tile", "ram_bwd_kernel_tile", "ram_last_error", "attn_bwd_prep",
                          "attn_bwd_chunk", "ring_attn_bwd_1gpu", "ring_attn_bwd_workspace_bytes",
                          "ring_attn_fwd_masks", "ring_attn_bwd_masks", "ring_attn_fwd_1gpu_noalloc",
                          "ram_mfma_probe", "ram_set_kernel_events"}, names
    for n in names:
        assert hasattr(lib, n), f"libram.so does not export {n}"


def test_kernel_events_validation(lib):
    assert lib.ram_set_kernel_events(FAKE, 0) == _lib.RAM_ERR_INVALID and "both" in _err(lib)
    assert lib.ram_set_kernel_events(0, FAKE) == _lib.RAM_ERR_INVALID
    assert lib.ram_set_kernel_events(0, 0) == _lib.RAM_OK


def test_mfma_probe_validation(lib):
    # rejected before any launch (no GPU needed)
    assert lib.ram_mfma_probe(0, 10, 1, FAKE2, 0) == _lib.RAM_ERR_INVALID
    assert lib.ram_mfma_probe(4, 0, 1, FAKE2, 0) == _lib.RAM_ERR_INVALID
    assert lib.ram_mfma_probe(4, 10, 2, FAKE2, 0) == _lib.RAM_ERR_INVALID
    assert lib.ram_mfma_probe(4, 10, 0, 0, 0) == _lib.RAM_ERR_INVALID


def _desc(**kw):
    d = dict(B=1, Sq=256, Skv=256, H=4, Hkv=2, D=128, dtype=ram.RAM_BF16, scale=0.125, softcap=0.0,
             causal=True, block_q=128, block_kv=64)
    d.update(kw)
    return ram.Desc(**d).c()


def _fdesc(**kw):
    """A descriptor at the forward tile of bf16 with D = 128 (128 x 64)."""
    return _desc(**kw)


def _src(**kw):
    return _lib.c_mask_src(kw.get("q_pos", 0), kw.get("kv_pos", 0), kw.get("q_pos_base", 0),
                           kw.get("kv_pos_base", 0), kw.get("q_seg", 0), kw.get("kv_seg", 0),
                           kw.get("q_meta_stride_b", 0), kw.get("kv_meta_stride_b", 0),
                           kw.get("dense", 0), kw.get("dense_ld", 0), kw.get("dense_chunk_step", 0))


def _bm(**kw):
    return _lib.c_block_mask(kw.get("tile_class", FAKE), kw.get("row_cnt", FAKE), kw.get("col_idx", FAKE),
                             kw.get("bits", 0), kw.get("col_cnt", 0), kw.get("row_idx", 0))


def _chunk(lib, d, *, q=FAKE, k=FAKE, v=FAKE, src=None, bm=None, sinks=0, mode=0, out=FAKE, lse=FAKE):
    src = src or _src()
    bm = bm or _bm()
    return lib.attn_fwd_chunk(ctypes.byref(d), q, k, v, ctypes.byref(src), ctypes.byref(bm), sinks, mode,
                              out, lse, 0)


def _err(lib):
    return lib.ram_last_error().decode()


def test_kernel_tile(lib):
    assert ram.kernel_tile(ram.RAM_BF16, 128) == (128, 64)
    assert ram.kernel_tile(ram.RAM_BF16, 64) == (128, 64)
    assert ram.kernel_tile(ram.RAM_F32, 64) == (128, 64)
    assert ram.kernel_tile(ram.RAM_F32, 128) == (128, 64)
    assert ram.bwd_kernel_tile(ram.RAM_BF16, 128) == (128, 64)
    assert ram.bwd_kernel_tile(ram.RAM_F32, 64) == (128, 64)
    with pytest.raises(ram.RamError) as e:
        ram.kernel_tile(ram.RAM_BF16, 96)
    assert e.value.status == _lib.RAM_ERR_UNSUPPORTED
    with pytest.raises(ram.RamError) as e:
        ram.kernel_tile(7, 128)
    assert e.value.status == _lib.RAM_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw, status, msg", [
    (dict(H=6, Hkv=4), _lib.RAM_ERR_INVALID, "multiple"),
    (dict(D=96), _lib.RAM_ERR_UNSUPPORTED, "head dim"),
    (dict(dtype=5), _lib.RAM_ERR_UNSUPPORTED, "dtype"),
    (dict(scale=0.0), _lib.RAM_ERR_INVALID, "scale"),
    (dict(scale=float("nan")), _lib.RAM_ERR_INVALID, "scale"),
    (dict(softcap=float("inf")), _lib.RAM_ERR_INVALID, "softcap"),
    (dict(causal=2), _lib.RAM_ERR_INVALID, "causal"),
    (dict(block_q=64), _lib.RAM_ERR_INVALID, "tile"),
    (dict(block_kv=128), _lib.RAM_ERR_INVALID, "tile"),
    (dict(B=-1), _lib.RAM_ERR_INVALID, "negative"),
    (dict(H=0), _lib.RAM_ERR_INVALID, ">= 1"),
    (dict(H=1 << 17, Hkv=1), _lib.RAM_ERR_UNSUPPORTED, "H=131072 above"),
    (dict(q_stride_b=100), _lib.RAM_ERR_INVALID, "q_stride_b"),
    (dict(kv_stride_b=256 * 2 * 128 + 3), _lib.RAM_ERR_INVALID, "kv_stride_b"),
])
def test_chunk_desc_validation(lib, kw, status, msg):
    assert _chunk(lib, _fdesc(**kw)) == status
    assert msg in _err(lib)


def test_chunk_pointer_validation(lib):
    d = _fdesc()
    assert _chunk(lib, d, q=0) == _lib.RAM_ERR_INVALID and "q is null" in _err(lib)
    assert _chunk(lib, d, k=FAKE + 2) == _lib.RAM_ERR_UNSUPPORTED and "aligned" in _err(lib)
    assert _chunk(lib, d, out=0) == _lib.RAM_ERR_INVALID
    assert _chunk(lib, d, lse=FAKE + 2) == _lib.RAM_ERR_INVALID
    assert _chunk(lib, d, mode=3) == _lib.RAM_ERR_INVALID and "mode" in _err(lib)
    assert _chunk(lib, d, src=_src(q_seg=FAKE)) == _lib.RAM_ERR_INVALID and "both" in _err(lib)
    assert _chunk(lib, d, src=_src(q_pos=FAKE + 1)) == _lib.RAM_ERR_INVALID
    assert _chunk(lib, d, src=_src(q_pos_base=2**31 - 10)) == _lib.RAM_ERR_INVALID and "overflow" in _err(lib)
    assert _chunk(lib, d, bm=_bm(row_cnt=0)) == _lib.RAM_ERR_INVALID and "row_cnt" in _err(lib)
    assert _chunk(lib, d, bm=_bm(col_idx=0)) == _lib.RAM_ERR_INVALID
    assert _chunk(lib, d, src=_src(kv_meta_stride_b=10)) == _lib.RAM_ERR_INVALID
    assert lib.attn_fwd_chunk(ctypes.byref(d), FAKE, FAKE, FAKE, None, ctypes.byref(_bm()), 0, 0, FAKE, FAKE,
                              0) == _lib.RAM_ERR_INVALID
    assert lib.attn_fwd_chunk(None, FAKE, FAKE, FAKE, None, None, 0, 0, FAKE, FAKE, 0) == _lib.RAM_ERR_INVALID


def test_ring_mask_layout(lib):
    # the ring's block masks sit at the offsets the workspace sizing lays out: classes, counts,
    # lists, then the bits when the forward needs them
    al = lambda x: (x + 255) // 256 * 256
    d = ram.Desc(B=1, Sq=4096, Skv=4096, H=8, Hkv=8, D=128)
    m = ram.ring_attn_fwd_masks(d, 4)
    acc = 4096 * 8 * 128 * 4
    tiles = 4 * 32 * 64
    assert (m["cls_off"], m["cnt_off"], m["col_off"], m["bits_off"], m["order_off"]) == (
        acc, acc + al(tiles), acc + al(tiles) + al(4 * 32 * 4), -1, -1)
    assert (m["block_q"], m["block_kv"], m["nQb"], m["nKb"], m["tile_words"]) == (128, 64, 32, 64, 256)
    mb = ram.ring_attn_fwd_masks(d, 4, ram.MaskSrc(dense=torch.zeros(1, dtype=torch.uint8)))
    assert mb["bits_off"] == m["col_off"] + tiles * 4
    assert mb["order_off"] == mb["bits_off"] + tiles * 256 * 4
    b = ram.ring_attn_bwd_masks(d, 4)
    assert b["bits_off"] == -1 and (b["block_q"], b["block_kv"], b["tile_words"]) == (128, 64, 256)
    assert b["cls_off"] > 0 and b["cnt_off"] == b["cls_off"] + al(tiles)
    with pytest.raises(ram.RamError):
        ram.ring_attn_fwd_masks(d, 0)
    with pytest.raises(ram.RamError):
        ram.ring_attn_bwd_masks(ram.Desc(B=1, Sq=64, Skv=64, H=3, Hkv=2, D=128), 2)


def test_noalloc_ring_rejects_shapes_past_its_scratch(lib):
    # the static scratch holds 64 MiB: a ring needing more is refused before anything runs
    big = _desc(B=1, Sq=32768, Skv=4096, H=32, Hkv=8)
    need = lib.ring_attn_workspace_bytes(ctypes.byref(big), 8, None)
    assert need > 64 << 20
    src = _src()
    st = lib.ring_attn_fwd_1gpu_noalloc(ctypes.byref(big), 8, -1, FAKE, FAKE, FAKE, ctypes.byref(src), 0, FAKE, FAKE2,
                                        0)
    assert st == _lib.RAM_ERR_UNSUPPORTED and "static scratch" in _err(lib) and str(need) in _err(lib)
    assert lib.ring_attn_fwd_1gpu_noalloc(None, 8, -1, FAKE, FAKE, FAKE, ctypes.byref(src), 0, FAKE, FAKE2,
                                          0) == _lib.RAM_ERR_INVALID


def test_mask_arrays_needed_only_with_kv_tiles(lib):
    # with key tiles, the classes and lists must be given; with Skv = 0 they may be null (the
    # kernels then read neither: covered on the GPU by test_empty_kv_null_mask_arrays)
    d = _fdesc()
    assert _chunk(lib, d, bm=_bm(tile_class=0)) == _lib.RAM_ERR_INVALID and "tile_class" in _err(lib)
    assert _chunk(lib, d, bm=_bm(col_idx=0)) == _lib.RAM_ERR_INVALID and "col_idx" in _err(lib)
    assert _chunk(lib, d, bm=_bm(row_cnt=0)) == _lib.RAM_ERR_INVALID and "row_cnt" in _err(lib)


def test_dense_mask_validation(lib):
    d = _fdesc()
    # a dense mask is applied through the tile bits: attention needs them
    assert _chunk(lib, d, src=_src(dense=FAKE2)) == _lib.RAM_ERR_INVALID and "tile bits" in _err(lib)
    assert _chunk(lib, d, src=_src(dense=FAKE2), bm=_bm(bits=FAKE + 4)) == _lib.RAM_ERR_INVALID
    assert "8-byte" in _err(lib)
    assert _chunk(lib, d, src=_src(dense=FAKE2, dense_ld=255), bm=_bm(bits=FAKE2)) == _lib.RAM_ERR_INVALID
    assert "dense_ld" in _err(lib)
    assert _chunk(lib, d, src=_src(dense=FAKE2, dense_chunk_step=-1), bm=_bm(bits=FAKE2)) == _lib.RAM_ERR_INVALID
    dm = _desc(block_q=64, block_kv=48)
    assert lib.build_block_mask(ctypes.byref(dm), ctypes.byref(_src(dense=FAKE2, dense_ld=100)),
                                ctypes.byref(_bm()), 0) == _lib.RAM_ERR_INVALID
    # the ring reads Skv + (n - 1) * step columns per row
    dr = _desc(B=1, Sq=512, Skv=512, H=4, Hkv=4)
    src = _src(dense=FAKE2, dense_chunk_step=512, dense_ld=4 * 512 - 1)
    assert _ring(lib, dr, 4, 3, src=src) == _lib.RAM_ERR_INVALID and "dense_ld" in _err(lib)
    src = _src(dense=FAKE2, dense_chunk_step=0, dense_ld=511)
    assert _ring(lib, dr, 4, 3, src=src) == _lib.RAM_ERR_INVALID
    # with a dense mask the ring workspace also holds the bits of every 128 x 64 tile (1 KiB each);
    # the bf16 D = 128 kernel needs them with key positions or segment IDs as well
    base = lib.ring_attn_workspace_bytes(ctypes.byref(dr), 4, None)
    plain = lib.ring_attn_workspace_bytes(ctypes.byref(dr), 4, ctypes.byref(_src()))
    dense = lib.ring_attn_workspace_bytes(ctypes.byref(dr), 4, ctypes.byref(_src(dense=FAKE2)))
    # (and, with any position, segment or dense array, the order of the rows of q tiles: 4 of them,
    # one 256-byte block)
    assert base == plain and dense == base + 4 * 4 * 8 * 1024 + 256
    assert lib.ring_attn_workspace_bytes(ctypes.byref(dr), 4, ctypes.byref(_src(kv_pos=FAKE2))) == dense
    assert lib.ring_attn_workspace_bytes(ctypes.byref(dr), 4, ctypes.byref(_src(q_pos=FAKE2))) == base + 256
    d64 = _desc(B=1, Sq=512, Skv=512, H=4, Hkv=4, D=64)
    b64 = lib.ring_attn_workspace_bytes(ctypes.byref(d64), 4, None)
    assert lib.ring_attn_workspace_bytes(ctypes.byref(d64), 4, ctypes.byref(_src(kv_pos=FAKE2))) == b64
    assert lib.ring_attn_workspace_bytes(ctypes.byref(d64), 4, ctypes.byref(_src(dense=FAKE2))) == b64 + 4 * 4 * 8 * 1024
    assert _ring(lib, dr, 4, 3, src=_src(dense=FAKE2), ws_bytes=dense - 1) == _lib.RAM_ERR_WORKSPACE


def test_empty_inputs_are_noops(lib):
    # B = 0 or Sq = 0: valid, nothing to do, nothing launched (works without a GPU)
    assert _chunk(lib, _fdesc(B=0), q=0, out=0, lse=0) == _lib.RAM_OK
    assert _chunk(lib, _fdesc(Sq=0), q=0, out=0, lse=0) == _lib.RAM_OK
    d = _desc(Sq=0)
    assert lib.build_block_mask(ctypes.byref(d), ctypes.byref(_src()), ctypes.byref(_bm()), 0) == _lib.RAM_OK
    assert lib.lse_merge(0, 5, 2, 128, 0, 0, 0, 0, 0) == _lib.RAM_OK
    assert _err(lib) == ""


def test_mask_validation(lib):
    bad = [dict(block_q=8), dict(block_kv=1024), dict(Skv=10_000_000, block_kv=16)]
    for kw in bad:
        d = _desc(**kw)
        st = lib.build_block_mask(ctypes.byref(d), ctypes.byref(_src()), ctypes.byref(_bm()), 0)
        assert st in (_lib.RAM_ERR_INVALID, _lib.RAM_ERR_UNSUPPORTED), kw
    d = _desc(block_q=256, block_kv=16)
    assert lib.build_block_mask(ctypes.byref(d), ctypes.byref(_src()), ctypes.byref(_bm(tile_class=0)),
                                0) == _lib.RAM_ERR_INVALID
    assert lib.build_block_mask(ctypes.byref(d), None, ctypes.byref(_bm()), 0) == _lib.RAM_ERR_INVALID


def test_merge_validation(lib):
    assert lib.lse_merge(1, 4, 2, 96, FAKE, FAKE, FAKE2, FAKE2, 0) == _lib.RAM_ERR_UNSUPPORTED
    assert lib.lse_merge(1, 4, 2, 128, FAKE, FAKE, FAKE, FAKE2, 0) == _lib.RAM_ERR_INVALID
    assert "alias" in _err(lib)
    assert lib.lse_merge(1, 4, 2, 128, 0, FAKE, FAKE2, FAKE2, 0) == _lib.RAM_ERR_INVALID
    assert lib.lse_merge(-1, 4, 2, 128, FAKE, FAKE, FAKE2, FAKE2, 0) == _lib.RAM_ERR_INVALID


def _ring(lib, d, n, r, ws=FAKE, ws_bytes=1 << 40, src=None, out=FAKE, q=FAKE):
    src = src or _src()
    return lib.ring_attn_fwd_1gpu(ctypes.byref(d), n, r, q, FAKE, FAKE, ctypes.byref(src), 0, out, FAKE2, ws,
                                  ws_bytes, 0)


def test_ring_validation_and_workspace(lib):
    al = lambda x: (x + 255) // 256 * 256
    d = _desc(B=1, Sq=4096, Skv=4096, H=8, Hkv=8)
    need = lib.ring_attn_workspace_bytes(ctypes.byref(d), 4, None)
    acc = 4096 * 8 * 128 * 4
    tiles = 4 * 32 * 64   # 4 chunks x 128-row tiles x 64-key tiles
    # 32 q tiles x 8 heads = 256 workgroups, under two per CU: room for the second half of a
    # split ring (its float32 result and lse)
    split = acc + 8 * 4096 * 4
    expect = acc + al(tiles) + al(4 * 32 * 4) + tiles * 4 + split
    assert need == expect
    # float32: accumulated in out, no split
    d32 = _desc(B=1, Sq=4096, Skv=4096, H=8, Hkv=8, dtype=ram.RAM_F32)
    assert lib.ring_attn_workspace_bytes(ctypes.byref(d32), 4, None) == need - acc - split
    # 64 q tiles x 8 heads = 512 workgroups: no split
    d2 = _desc(B=2, Sq=4096, Skv=4096, H=8, Hkv=8)
    tiles2 = 4 * 64 * 64
    assert lib.ring_attn_workspace_bytes(ctypes.byref(d2), 4, None) == (
        2 * acc + al(tiles2) + al(4 * 64 * 4) + tiles2 * 4)
    # Sq * H / Hkv >= 32768 without a cap: V of every chunk also rearranged for the kernel, in
    # tiles of 32 keys x 128 dims (8 KiB) per kv head, a ragged chunk rounded up to 32 keys
    d3 = _desc(B=1, Sq=32768, Skv=4000, H=32, Hkv=8)
    acc3, tiles3 = 32768 * 32 * 128 * 4, 8 * 256 * 63
    base3 = acc3 + al(tiles3) + al(8 * 256 * 4) + al(tiles3 * 4)
    assert lib.ring_attn_workspace_bytes(ctypes.byref(d3), 8, None) == base3 + 8 * 8 * 125 * 8192
    d3c = _desc(B=1, Sq=32768, Skv=4000, H=32, Hkv=8, softcap=50.0)
    assert lib.ring_attn_workspace_bytes(ctypes.byref(d3c), 8, None) == base3
    assert _ring(lib, d, 65536, -1) == _lib.RAM_ERR_UNSUPPORTED and "65535" in _err(lib)
    assert lib.ring_attn_workspace_bytes(ctypes.byref(d), 0, None) == 0
    assert _ring(lib, d, 0, -1) == _lib.RAM_ERR_INVALID
    assert _ring(lib, d, 4, 4) == _lib.RAM_ERR_INVALID and "q_shard" in _err(lib)
    assert _ring(lib, d, 4, -2) == _lib.RAM_ERR_INVALID
    assert _ring(lib, d, 4, 3, ws_bytes=need - 1) == _lib.RAM_ERR_WORKSPACE and "need" in _err(lib)
    assert _ring(lib, d, 4, 3, ws=FAKE + 16) == _lib.RAM_ERR_WORKSPACE
    assert _ring(lib, d, 4, 3, ws=0) == _lib.RAM_ERR_WORKSPACE
    assert _ring(lib, d, 4, 3, src=_src(q_pos_base=2**31 - 5000)) == _lib.RAM_ERR_INVALID  # 3*Sq overflows
    assert _ring(lib, d, 4, 3, src=_src(kv_meta_stride_b=4096)) == _lib.RAM_ERR_INVALID    # must span 4 chunks
    assert _ring(lib, d, 4, 3, out=0) == _lib.RAM_ERR_INVALID
    # the bf16 D = 128 forward addresses one chunk's key rows with 32-bit byte offsets
    big = _desc(B=1, Sq=4096, Skv=524288, H=32, Hkv=32)
    assert _ring(lib, big, 2, 1) == _lib.RAM_ERR_UNSUPPORTED and "4 GiB" in _err(lib)
    assert _chunk(lib, _fdesc(Skv=524288, H=32, Hkv=32, block_q=128)) == _lib.RAM_ERR_UNSUPPORTED
    # the ring picks its own tile: a caller's block_q/block_kv are ignored
    dt = _desc(B=1, Sq=4096, Skv=4096, H=8, Hkv=8, block_q=32, block_kv=32)
    assert lib.ring_attn_workspace_bytes(ctypes.byref(dt), 4, None) == need
    assert _ring(lib, _desc(B=0), 4, 3, q=0, out=0) == _lib.RAM_OK


def test_binding_rejects_cpu_tensors(lib):
    import torch
    d = ram.Desc(B=1, Sq=8, Skv=8, H=1, Hkv=1, D=64, dtype=ram.RAM_F32, scale=0.1)
    x = torch.zeros(8 * 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        ram.attn_fwd_chunk(d, x, x, x, ram.MaskSrc(), ram.alloc_block_mask(d, device="cpu"), None, 0, x,
                           torch.zeros(8), stream=0)


def test_backward_validation(lib):
    d = _desc()
    z = ctypes.c_void_p(0)
    args = lambda **kw: (ctypes.byref(kw.get("d", d)), kw.get("q", FAKE), kw.get("k", FAKE), kw.get("v", FAKE),
                         kw.get("dout", FAKE), kw.get("lse", FAKE2), kw.get("delta", FAKE2),
                         ctypes.byref(kw.get("src", _src())), ctypes.byref(kw.get("bm", _bm(col_cnt=FAKE, row_idx=FAKE))),
                         kw.get("mode", 0), kw.get("dq", FAKE), kw.get("dk", FAKE), kw.get("dv", FAKE), 0)
    # built for bf16 and float32, D = 64 and 128 only
    assert lib.attn_bwd_chunk(*args(d=_desc(D=32))) == _lib.RAM_ERR_UNSUPPORTED
    assert lib.attn_bwd_chunk(*args(d=_desc(D=96))) == _lib.RAM_ERR_UNSUPPORTED
    assert lib.attn_bwd_chunk(*args(d=_desc(dtype=5))) == _lib.RAM_ERR_UNSUPPORTED
    # the transposed lists are required, both or neither
    assert lib.attn_bwd_chunk(*args(bm=_bm())) == _lib.RAM_ERR_INVALID and "transposed" in _err(lib)
    assert lib.attn_bwd_chunk(*args(bm=_bm(col_cnt=FAKE))) == _lib.RAM_ERR_INVALID and "both" in _err(lib)
    assert lib.attn_bwd_chunk(*args(mode=2)) == _lib.RAM_ERR_INVALID and "dq_mode" in _err(lib)
    assert lib.attn_bwd_chunk(*args(dout=FAKE + 2)) == _lib.RAM_ERR_UNSUPPORTED
    assert lib.attn_bwd_chunk(*args(delta=0)) == _lib.RAM_ERR_INVALID
    assert lib.attn_bwd_chunk(*args(dk=0)) == _lib.RAM_ERR_INVALID
    assert lib.attn_bwd_chunk(*args(src=_src(dense=FAKE2))) == _lib.RAM_ERR_INVALID and "bits" in _err(lib)
    # prep: sinks need dsinks
    assert lib.attn_bwd_prep(ctypes.byref(d), FAKE, FAKE, FAKE2, FAKE2, FAKE2, z, 0) == _lib.RAM_ERR_INVALID
    assert lib.attn_bwd_prep(ctypes.byref(_desc(D=96)), FAKE, FAKE, FAKE2, 0, FAKE2, 0, 0) == _lib.RAM_ERR_UNSUPPORTED
    assert lib.attn_bwd_prep(ctypes.byref(_desc(dtype=5)), FAKE, FAKE, FAKE2, 0, FAKE2, 0,
                             0) == _lib.RAM_ERR_UNSUPPORTED
    # the ring: workspace holds float32 dq, dk, dv, delta and the masks with transposed lists
    dr = _desc(B=1, Sq=512, Skv=512, H=4, Hkv=2)
    need = lib.ring_attn_bwd_workspace_bytes(ctypes.byref(dr), 4, None)
    al = lambda x: (x + 255) // 256 * 256
    tiles = 4 * 4 * 8
    # the dk / dv launch of a chunk has 2 kv heads x 8 kv tiles = 16 workgroups: the 2 heads of
    # each group go to 2 workgroups, whose partial dk and dv for one chunk take 2 x 2 x 512 x 2 x 128 floats
    parts = 2 * al(2 * 512 * 2 * 128 * 4)
    expect = (al(512 * 4 * 128 * 4) + 2 * al(4 * 512 * 2 * 128 * 4) + al(2 * 4 * 512 * 4) + al(tiles)
              + al(4 * 4 * 4) + al(tiles * 4) + al(4 * 8 * 4) + al(tiles * 4) + parts)
    assert need == expect
    # float32 runs one workgroup per kv tile: no partial sums
    f32 = lib.ring_attn_bwd_workspace_bytes(ctypes.byref(_desc(B=1, Sq=512, Skv=512, H=4, Hkv=2, dtype=ram.RAM_F32)), 4,
                                            None)
    assert f32 == expect - parts
    dense = lib.ring_attn_bwd_workspace_bytes(ctypes.byref(dr), 4, ctypes.byref(_src(dense=FAKE2)))
    assert dense == need + tiles * 1024
    assert lib.ring_attn_bwd_workspace_bytes(ctypes.byref(_desc(D=96)), 4, None) == 0
    d64 = _desc(B=1, Sq=512, Skv=512, H=4, Hkv=2, D=64)
    assert lib.ring_attn_bwd_workspace_bytes(ctypes.byref(d64), 4, None) == expect - parts - (
        al(512 * 4 * 128 * 4) + 2 * al(4 * 512 * 2 * 128 * 4)) + al(512 * 4 * 64 * 4) + 2 * al(4 * 512 * 2 * 64 * 4) + (
        2 * al(2 * 512 * 2 * 64 * 4))
    ring = lambda ws_bytes, **kw: lib.ring_attn_bwd_1gpu(
        ctypes.byref(kw.get("d", dr)), 4, kw.get("r", 3), FAKE, FAKE, FAKE, FAKE, FAKE2, FAKE,
        ctypes.byref(_src()), kw.get("sinks", 0), FAKE, FAKE, FAKE, kw.get("dsinks", 0), FAKE, ws_bytes, 0)
    assert ring(need - 1) == _lib.RAM_ERR_WORKSPACE and "need" in _err(lib)
    assert ring(need, r=4) == _lib.RAM_ERR_INVALID
    assert ring(need, sinks=FAKE2) == _lib.RAM_ERR_INVALID and "dsinks" in _err(lib)
