"""Static check of the compiled kernels: no instruction touches the destination registers of an
LDS read before the `s_waitcnt lgkmcnt` that covers that read.

Several kernels issue LDS reads from inline assembly and wait for them later, so the compiler
does not know that the registers are written asynchronously; if it copies such a value (for
example to join the results of reads issued in two branches) before the wait, it copies whatever
the register held before the read. This test compiles every kernel source to gfx950 assembly
and scans each function's instructions in program order, keeping the LDS reads still in flight
(an `lgkmcnt(n)` wait leaves the newest n; a wait with n = 0 clears them). LDS reads complete
in order, so a later LDS read writing the same register is not flagged. The scan follows the
text order through branches, which is conservative for these kernels (no false reports on the
current sources).
"""
import concurrent.futures
import glob
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from ring_attention_merge_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ring_attention_merge_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _regs(op):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", op)
    return {int(m.group(1))} if m else set()


def lds_hazards(asm: str):
    """(function, instruction, LDS read) triples where the instruction reads or overwrites the
    read's destination before a wait covers it."""
    found = []
    for fn in re.findall(r"^\s*\.type\s+(_Z\w+),@function", asm, re.M):
        body = asm[asm.index("\n" + fn + ":") + 1:]
        body = body[: body.index(".Lfunc_end")]
        lines = [l.split(";")[0].strip() for l in body.split("\n")]
        lines = [l for l in lines if l and not l.startswith(".")]
        pending = []   # (instruction, destination registers), oldest first
        for l in lines:
            parts = l.replace(",", " ").split()
            op, ops = parts[0], parts[1:]
            if op.startswith("s_waitcnt") and "lgkmcnt" in l:
                n = int(re.search(r"lgkmcnt\((\d+)\)", l).group(1))
                pending = pending[len(pending) - n:] if n else []
                continue
            writes = not op.startswith(("ds_write", "buffer", "global_store", "s_"))
            dst = _regs(ops[0]) if ops and writes else set()
            srcs = set()
            for o in (ops[1:] if dst else ops):
                srcs |= _regs(o)
            touched = srcs | (set() if op.startswith("ds_read") else dst)
            for (src_l, r) in pending:
                if touched & r:
                    found.append((fn, l, src_l))
            if op.startswith("ds_read"):
                pending.append((l, _regs(ops[0])))
            elif op.startswith(("ds_", "s_load", "s_buffer_load")):
                pending.append((l, set()))   # counts towards lgkmcnt, no result tracked
    return found


def _compile(src, out_dir):
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    # the flags libram.so is built with
    flags = [f for f in build.HIP_FLAGS if f not in ("-fPIC",)]
    cmd = [HIPCC, *flags, "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{src}: {r.stderr[-2000:]}"
    return src, open(out).read()


def test_checker_flags_an_early_copy():
    """A copy of an LDS result before its wait is reported; after the wait it is not."""
    early = """\t.type\t_Zfoo,@function
_Zfoo:
\tds_read_b128 v[4:7], v1
\tv_mov_b32_e32 v9, v5
\ts_waitcnt lgkmcnt(0)
.Lfunc_end0:
"""
    late = early.replace("\tv_mov_b32_e32 v9, v5\n\ts_waitcnt lgkmcnt(0)\n", "\ts_waitcnt lgkmcnt(0)\n\tv_mov_b32_e32 v9, v5\n")
    partial = """\t.type\t_Zfoo,@function
_Zfoo:
\tds_read_b128 v[4:7], v1
\tds_read_b128 v[8:11], v1 offset:16
\ts_waitcnt lgkmcnt(1)
\tv_mov_b32_e32 v20, v4
\tv_mov_b32_e32 v21, v8
.Lfunc_end0:
"""
    assert len(lds_hazards(early)) == 1
    assert lds_hazards(late) == []
    assert [h[1] for h in lds_hazards(partial)] == ["v_mov_b32_e32 v21, v8"]


_ASM = {}


def _all_asm():
    """gfx950 assembly of every kernel source (compiled once per test session)."""
    if not _ASM:
        sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
        assert sources
        with tempfile.TemporaryDirectory() as d:
            with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
                _ASM.update(ex.map(lambda s: _compile(s, d), sources))
    return sorted(_ASM.items())


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not available")
def test_no_packed_fp32_instructions():
    """The device code holds no packed fp32 arithmetic (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32):
    the build turns the feature off for every kernel source."""
    bad = []
    for src, asm in _all_asm():
        bad += [f"{os.path.basename(src)}: {m}" for m in re.findall(r"\bv_pk_(?:add|mul|fma)_f32\b[^\n]*", asm)]
    assert not bad, "\n".join(bad[:20])


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not available")
def test_no_lds_result_read_before_its_wait():
    results = _all_asm()
    bad = []
    for src, asm in results:
        bad += [f"{os.path.basename(src)}: {fn[:60]}: '{ins}' before the wait of '{rd}'"
                for fn, ins, rd in lds_hazards(asm)]
    assert not bad, "\n".join(bad[:20])
