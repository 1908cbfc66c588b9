"""Code generation checks on the gfx950 assembly of every kernel source (CPU only: hipcc -S).

A VMEM store with more than 64 bits of data reads its data registers after issue; a VALU
instruction that overwrites one of them right behind the store made the store write the new
value for some lanes (seen as torn chunk records). The kernels therefore store at most 8 bytes
per instruction. The compiler merges plain 8-byte stores to adjacent addresses into one 16-byte
store, so the kernels use the buffer-store intrinsics, which it leaves alone; these tests keep
any wide store, and in particular one followed closely by a write of its data registers, out of
the library.

The forward kernels are also checked for a wait on all outstanding loads right behind a load,
the pattern a load under a branch or a conversion next to a load produces.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunked_kimi_delta_amd", "csrc")

WIDE_STORE = re.compile(r"^(global_store_dwordx[34]|buffer_store_dwordx[34]|flat_store_dwordx[34])\s+(.*)")


def vregs(tok: str) -> set:
    out = set()
    for m in re.finditer(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]", tok):
        if m.group(1):
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def wide_store_overwrites(asm: str, window: int = 3):
    """(line, store, writer) for every wide store whose data registers a VALU instruction among
    the next `window` instructions writes."""
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    instr = [(i, l) for i, l in enumerate(lines)
             if l and not l.endswith(":") and not l.startswith(".")]
    hits = []
    for k, (i, l) in enumerate(instr):
        m = WIDE_STORE.match(l)
        if not m:
            continue
        ops = [x.strip() for x in m.group(2).split(",")]
        data = vregs(ops[0]) if m.group(1).startswith("buffer") else vregs(ops[1])
        for _, nxt in instr[k + 1:k + 1 + window]:
            if nxt.startswith("v_") and not nxt.startswith(("v_cmp", "v_readfirstlane",
                                                            "v_readlane")):
                parts = nxt.split(None, 1)
                if len(parts) == 2 and vregs(parts[1].split(",")[0]) & data:
                    hits.append((i, l, nxt))
                    break
    return hits


def test_detector_finds_the_pattern():
    asm = """
    buffer_store_dwordx4 v[52:55], v101, s[20:23], s6 offen
    v_mov_b32_e32 v52, 0
    global_store_dwordx4 v[2:3], v[8:11], off
    v_add_f32_e32 v1, v2, v3
    buffer_store_dwordx2 v[4:5], v1, s[0:3], 0 offen
    v_mov_b32_e32 v4, 0
    """
    hits = wide_store_overwrites(asm)
    assert [h[2] for h in hits] == ["v_mov_b32_e32 v52, 0"]


def _asm(src: str, out_dir: str) -> str:
    import sys
    sys.path.insert(0, os.path.join(ROOT, "chunked_kimi_delta_amd"))
    from build import HIPCC_FLAGS, hipcc
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    subprocess.run([hipcc()] + HIPCC_FLAGS + ["--cuda-device-only", "-S", src, "-o", out],
                   check=True, capture_output=True)
    return open(out).read()


_ASMS = {}


def kernel_asms():
    if not _ASMS:
        srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
        with tempfile.TemporaryDirectory() as d, cf.ThreadPoolExecutor(4) as ex:
            _ASMS.update(zip(srcs, ex.map(lambda s: _asm(s, d), srcs)))
    return _ASMS


HAVE_HIPCC = shutil.which("hipcc") is not None or os.path.exists("/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not HAVE_HIPCC, reason="hipcc not available")
def test_no_wide_store_data_overwrite_in_kernels():
    bad = {os.path.basename(s): wide_store_overwrites(a)[:3] for s, a in kernel_asms().items()}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, bad


@pytest.mark.skipif(not HAVE_HIPCC, reason="hipcc not available")
def test_no_wide_stores_at_all():
    bad = {}
    for s, a in kernel_asms().items():
        n = sum(1 for l in a.splitlines() if WIDE_STORE.match(l.split(";")[0].strip()))
        if n:
            bad[os.path.basename(s)] = n
    assert not bad, f"stores wider than 8 bytes: {bad}"


def load_then_full_wait(asm: str, window: int = 3):
    """(line, load) pairs where `s_waitcnt vmcnt(0)` follows a vector-memory load within
    `window` instructions: the wave waits for every load it has in flight right after issuing
    one, which serialises a load phase into memory round trips."""
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    ins = [(i, l) for i, l in enumerate(lines) if l and not l.startswith(".") and not l.endswith(":")]
    out = []
    for n, (i, l) in enumerate(ins):
        # a kernel's deliberate drain (vm_drain: "vmcnt(0) expcnt(6)") is not this pattern
        if l.startswith("s_waitcnt") and "vmcnt(0)" in l and "expcnt(6)" not in l:
            for _, p in ins[max(0, n - window):n]:
                if re.match(r"(global|buffer|flat)_load", p):
                    out.append((i, p))
                    break
    return out


def test_detector_finds_a_load_then_full_wait():
    asm = "\n".join(["global_load_ushort v1, v[2:3], off", "v_mov_b32 v5, 0",
                     "s_waitcnt vmcnt(0)", "v_lshlrev_b32_e32 v1, 16, v1"])
    assert len(load_then_full_wait(asm)) == 1
    assert load_then_full_wait(asm.replace("vmcnt(0)", "vmcnt(3)")) == []
    assert load_then_full_wait(asm.replace("vmcnt(0)", "vmcnt(0) expcnt(6)")) == []


# Forward kernels: their loads are issued unconditionally and converted where they are used,
# so no load is waited for on the spot (a load under a per-row branch, or a conversion next to
# it, had serialised the prepare and token-recurrence load phases).
FORWARD_SOURCES = ("kda_prepare32.hip", "kda_state32.hip", "kda_state64.hip",
                   "kda_recurrent.hip", "kda_prepare.hip", "kda_state.hip")


@pytest.mark.skipif(not HAVE_HIPCC, reason="hipcc not available")
def test_forward_kernels_do_not_wait_on_each_load():
    bad = {}
    for s, a in kernel_asms().items():
        if os.path.basename(s) in FORWARD_SOURCES:
            hits = load_then_full_wait(a)
            if hits:
                bad[os.path.basename(s)] = hits[:3]
    assert not bad, bad


# One matrix-core product taking the result of a product of another shape as its accumulator
# (SrcC) a few instructions later. Copies of the state kernel with a 16x16x16 result feeding a
# 16x16x32 accumulator 3-8 instructions later, or a 16x16x32 result feeding a 16x16x16
# accumulator in place 4-6 instructions later, computed wrong sums for those accumulators (o
# off by 0.14-0.8 relative), while products of one shape chained back to back were always
# right. The compiler's wait between two shapes is evidently too short on gfx950, so the
# library keeps such pairs out (the state kernels form -U and the Mqk term with 16x16x32
# products, zero-padded).
MFMA = re.compile(r"^(v_mfma_\S+)\s+(.*)")


def mfma_cross_shape_accumulator(asm: str, window: int = 12):
    """(line, producer, consumer) for every v_mfma whose destination a v_mfma of another
    opcode reads as SrcC within `window` instructions (registers rewritten in between end the
    dependence)."""
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    ins = [(i, l) for i, l in enumerate(lines) if l and not l.startswith(".") and not l.endswith(":")]
    hits = []
    for k, (i, l) in enumerate(ins):
        m = MFMA.match(l)
        if not m:
            continue
        live = vregs(m.group(2).split(",")[0])      # registers still holding the product
        for _, nxt in ins[k + 1:k + 1 + window]:
            m2 = MFMA.match(nxt)
            if m2 and m2.group(1) != m.group(1):
                ops = [x.strip() for x in m2.group(2).split(",")]
                if len(ops) > 3 and vregs(ops[3]) & live:
                    hits.append((i, l, nxt))
                    break
            parts = nxt.split(None, 1)
            if len(parts) == 2 and nxt.startswith("v_"):
                live -= vregs(parts[1].split(",")[0])
            if not live:
                break
    return hits


def test_detector_finds_a_cross_shape_accumulator():
    asm = "\n".join(["v_mfma_f32_16x16x16_f16 v[24:27], v[20:21], v[66:67], 0",
                     "s_add_i32 s0, s23, s0",
                     "v_mfma_f32_16x16x32_f16 v[24:27], v[42:45], v[28:31], v[24:27]",
                     "v_mfma_f32_16x16x32_f16 v[4:7], v[8:11], v[12:15], v[4:7]"])
    assert len(mfma_cross_shape_accumulator(asm)) == 1
    # one shape chained: no hit
    assert mfma_cross_shape_accumulator(asm.replace("16x16x16_f16", "16x16x32_f16")) == []
    # the other direction, in place
    rev = "\n".join(["v_mfma_f32_16x16x32_f16 v[10:13], v[10:13], v[46:49], v[18:21]",
                      "v_cvt_pk_bf16_f32 v22, v38, s0",
                      "v_mfma_f32_16x16x16_f16 v[10:13], v[76:77], v[50:51], v[10:13]"])
    assert len(mfma_cross_shape_accumulator(rev)) == 1
    # the product's registers rewritten before the other shape reads them: no dependence
    rewritten = asm.replace("s_add_i32 s0, s23, s0", "v_mov_b32_e32 v[24:27], 0")
    assert mfma_cross_shape_accumulator(rewritten) == []


@pytest.mark.skipif(not HAVE_HIPCC, reason="hipcc not available")
def test_no_cross_shape_mfma_accumulator_in_kernels():
    bad = {os.path.basename(s): mfma_cross_shape_accumulator(a)[:3]
           for s, a in kernel_asms().items()}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, bad
