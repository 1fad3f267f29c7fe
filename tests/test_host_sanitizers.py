"""Plan lifecycle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds tests/host_sanitize_driver.cpp with the mask compiler (plan.cpp) and
the descriptor plan cache (desc_cache.cpp) using g++ with ASan, UBSan and the
libstdc++ container annotations, and runs it.  The driver creates, inspects
(every blob byte and layout section) and destroys plans for every mask family
and bitmap layout over several shapes, drives every invalid-argument class,
and cycles the descriptor cache past its capacity with host stand-ins for the
three GPU entry points.  Any out-of-bounds access, use after free, leak or
undefined behaviour fails the run.  A second build under ThreadSanitizer
runs the driver's threaded mode: four threads sharing the descriptor cache
(lookups, uploads, launches, releases, clears), creating plans and reading
their thread-local error strings.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_masked_amd", "csrc")


def _build(tmp_path, name, sanitize_flags):
    exe = str(tmp_path / name)
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *sanitize_flags]
    cmd = ["g++", *flags, f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "desc_cache.cpp"),
           "-o", exe, "-lpthread"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:]
    return exe


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_plan_lifecycle_is_clean_under_asan_and_ubsan(tmp_path):
    exe = _build(tmp_path, "driver_asan", ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                           "-D_GLIBCXX_SANITIZE_VECTOR"])
    # verify_asan_link_order=0: the process may carry a preloaded library of
    # its environment ahead of the sanitizer runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "all plan lifecycles clean" in r.stdout
    assert "runtime error" not in r.stdout, r.stdout[-4000:]


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_descriptor_cache_is_race_free_under_tsan(tmp_path):
    exe = _build(tmp_path, "driver_tsan", ["-fsanitize=thread"])
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe, "threads"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "threads clean" in r.stdout
    assert "ThreadSanitizer" not in r.stdout, r.stdout[-4000:]
