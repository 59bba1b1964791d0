"""Generated-code guard for the gfx950 kernels (CPU only: hipcc cross-compiles).

A vector-memory store of more than 8 bytes keeps reading its data registers
for a while after it issues.  If the very next instruction is a VALU write to
one of those registers, the store can send the new value.  The compiler inserts
a wait state for global stores.  On gfx950 it inserts none for buffer stores
that take an SGPR offset, and 16-byte bf16 outputs were seen to lose their
first dword that way.  This test compiles every kernel source to gfx950
assembly and fails on any wide store whose next instruction overwrites its
data.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from linear_recurrence_scans_amd import build as B

HIPCC = B.HIPCC
KERNEL_SOURCES = [s for s in B.SOURCES + B.BENCH_SOURCES if s != "api.hip"]

pytestmark = pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                                reason="hipcc not available")

WIDE_STORE = re.compile(r"^(global|buffer|flat)_store_dwordx([34])\b")
VALU_DEST = re.compile(r"^v_\w+\s+v(?:\[(\d+):(\d+)\]|(\d+))\b")


def _asm(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    cmd = [HIPCC] + B.FLAGS + ["--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


def _store_data_regs(line):
    """VGPR range holding a wide store's data."""
    regs = re.findall(r"v\[(\d+):(\d+)\]", line)
    if line.startswith("buffer_"):
        lo, hi = regs[0]        # buffer_store vdata, voffset, srsrc, soffset
    else:
        lo, hi = regs[-1]       # global_store vaddr, vdata, saddr
    return int(lo), int(hi)


def _hazards(asm_text):
    lines = [l.strip() for l in asm_text.splitlines()]
    lines = [l for l in lines if l and not l.startswith((";", ".")) and not l.endswith(":")]
    found = []
    for i, l in enumerate(lines[:-1]):
        if not WIDE_STORE.match(l):
            continue
        lo, hi = _store_data_regs(l)
        m = VALU_DEST.match(lines[i + 1])
        if not m:
            continue
        d_lo = int(m.group(1) or m.group(3))
        d_hi = int(m.group(2) or m.group(3))
        if d_lo <= hi and lo <= d_hi:
            found.append((l, lines[i + 1]))
    return found


def test_scanner_flags_the_pattern():
    """The scanner itself: a wide store followed by a write of its data."""
    bad = "buffer_store_dwordx4 v[10:13], v1, s[4:7], s8 offen nt\nv_cvt_pk_bf16_f32 v10, v20, v21\n"
    ok = "buffer_store_dwordx4 v[10:13], v1, s[4:7], s8 offen nt\ns_nop 0\nv_cvt_pk_bf16_f32 v10, v20, v21\n"
    glob = "global_store_dwordx4 v[2:3], v[10:13], off nt\nv_mov_b32 v12, 0\n"
    other = "global_store_dwordx4 v[2:3], v[10:13], off nt\nv_mov_b32 v14, 0\n"
    assert len(_hazards(bad)) == 1
    assert _hazards(ok) == []
    assert len(_hazards(glob)) == 1
    assert _hazards(other) == []


def test_no_wide_store_data_overwrite():
    tmp = tempfile.mkdtemp(prefix="miscan_asm_")
    try:
        with cf.ThreadPoolExecutor(max_workers=len(KERNEL_SOURCES)) as ex:
            outs = list(ex.map(lambda s: _asm(s, tmp), KERNEL_SOURCES))
        problems = {}
        n_wide = 0
        for src, path in zip(KERNEL_SOURCES, outs):
            text = open(path).read()
            n_wide += sum(1 for l in text.splitlines() if WIDE_STORE.match(l.strip()))
            h = _hazards(text)
            if h:
                problems[src] = h[:3]
        assert n_wide > 0, "no wide stores found: the scanner no longer matches the code"
        assert not problems, problems
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
