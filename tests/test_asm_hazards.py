"""Compiled-code check of the transposed LDS reads (CPU; needs hipcc).

build() compiles fwd.hip and bwd.hip to gfx950 assembly as well and refuses
to link when an instruction names a destination register of a transposed
LDS read before its lgkmcnt(0) wait (long_context_masked_amd._build,
uses_of_pending_reads).  These tests check the scan on planted text and
run it on the current sources with the library's flags.
"""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from long_context_masked_amd import _build as B
from long_context_masked_amd._build import scan_transposed_reads, uses_of_pending_reads

SOURCES = B.TR_READ_SOURCES


def test_scan_flags_a_planted_reuse():
    """The scan itself: a register reused before the wait is reported, the
    same use after the wait is not; build()'s check raises on it."""
    bad = ("_ZN3lcm1kEv:\n\tds_read_b64_tr_b16 v[4:5], v1 offset:0\n"
           "\tv_fma_f32 v5, v6, s2, v7\n\ts_waitcnt lgkmcnt(0)\n\ts_endpgm\n")
    good = ("_ZN3lcm1kEv:\n\tds_read_b64_tr_b16 v[4:5], v1 offset:0\n"
            "\tv_fma_f32 v8, v6, s2, v7\n\ts_waitcnt lgkmcnt(0)\n\tv_mov_b32 v9, v5\n\ts_endpgm\n")
    assert len(uses_of_pending_reads(bad)) == 1
    assert uses_of_pending_reads(good) == []
    with pytest.raises(RuntimeError, match="in-flight"):
        scan_transposed_reads({"bad.hip": bad})
    scan_transposed_reads({"good.hip": good})


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
            results = dict(ex.map(compile_one, SOURCES))
    scan_transposed_reads(results)
