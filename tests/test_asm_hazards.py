"""Compiled-code check of the transposed LDS reads (CPU; needs hipcc).

The kernels issue ds_read_b64_tr_b16 as inline assembly and wait for it with
an explicit s_waitcnt lgkmcnt(0) that names the destination registers.  The
compiler takes an asm output as written when the instruction issues, so
under register pressure it may spill such a register, copy it, or reuse it
as a temporary before the data has arrived; the read then lands on top of
other values, or the kernel consumes stale data.  Nothing in the source
prevents this: it depends on the register allocation of each build.  This
test compiles the two kernel sources with the library's own flags and scans
the gfx950 assembly: between a transposed read and the next lgkmcnt(0) wait,
no instruction may name any of its destination registers.  (A linear scan of
each kernel's text; the reads and their waits sit in straight-line code.)
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from long_context_masked_amd import _build as B

SOURCES = ["fwd.hip", "bwd.hip"]


def _vregs(operand):
    m = re.match(r"v\[(\d+):(\d+)\]$", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", operand)
    return {int(m.group(1))} if m else set()


def uses_of_pending_reads(asm_text):
    """(kernel, line, instruction) for every instruction that names a register
    whose transposed LDS read has not yet been waited for."""
    found, pending, kernel = [], set(), None
    for n, line in enumerate(asm_text.split("\n"), 1):
        t = line.strip()
        m = re.match(r"^(_Z\w+):", t)
        if m:
            kernel, pending = m.group(1), set()
            continue
        if not t or t.startswith((";", ".")):
            continue
        parts = t.split(None, 1)
        op = parts[0]
        operands = [a.strip().split()[0] for a in parts[1].split(",") if a.strip()] if len(parts) > 1 else []
        if op == "ds_read_b64_tr_b16":
            pending |= _vregs(operands[0])
            continue
        if op == "s_endpgm" or (op == "s_waitcnt" and "lgkmcnt(0)" in t):
            pending = set()
            continue
        if pending and any(_vregs(a) & pending for a in operands):
            found.append((kernel, n, t))
    return found


def test_scan_flags_a_planted_reuse():
    """The scan itself: a register reused before the wait is reported, the
    same use after the wait is not."""
    bad = ("_ZN3lcm1kEv:\n\tds_read_b64_tr_b16 v[4:5], v1 offset:0\n"
           "\tv_fma_f32 v5, v6, s2, v7\n\ts_waitcnt lgkmcnt(0)\n\ts_endpgm\n")
    good = ("_ZN3lcm1kEv:\n\tds_read_b64_tr_b16 v[4:5], v1 offset:0\n"
            "\tv_fma_f32 v8, v6, s2, v7\n\ts_waitcnt lgkmcnt(0)\n\tv_mov_b32 v9, v5\n\ts_endpgm\n")
    assert len(uses_of_pending_reads(bad)) == 1
    assert uses_of_pending_reads(good) == []


@pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None, reason="hipcc not found")
def test_no_register_of_an_inflight_transposed_read_is_touched():
    with tempfile.TemporaryDirectory() as tmp:
        def compile_one(src):
            out = os.path.join(tmp, src + ".s")
            cmd = [B.HIPCC, *B.HIP_FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
            r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
            assert r.returncode == 0, r.stdout[-2000:]
            return src, open(out).read()

        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            results = list(ex.map(compile_one, SOURCES))
    for src, text in results:
        assert "ds_read_b64_tr_b16" in text, f"{src}: no transposed reads compiled"
        found = uses_of_pending_reads(text)
        assert not found, f"{src}: {len(found)} uses of in-flight transposed reads, e.g. " + \
            "; ".join(f"{k} line {n}: {i}" for k, n, i in found[:3])
