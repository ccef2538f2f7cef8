"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

abi.cpp is rebuilt with both sanitizers on its host pass (the kernels as usual) and the
whole CPU ABI suite (tests/test_abi_cpu.py: every argument check, the gate and its measured
table, workspace sizes) runs against that build in a child process that preloads the
sanitizer runtime. Any out-of-bounds access, use after free or undefined behaviour there
ends the child with a report and fails this test. No GPU is needed: every call the suite
makes is rejected or answered before the library reaches the HIP runtime.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import ctypes, sys
sys.path.insert(0, {root!r})
from block_fp8_mixture_top_amd import _lib as L
L.load({lib!r})
assert hasattr(ctypes.CDLL(None), "__asan_init"), "the sanitizer runtime is not loaded"
import pytest
sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider", {suite!r}]))  # -s: reports reach stderr
"""


def test_abi_suite_under_host_sanitizers(tmp_path):
    from block_fp8_mixture_top_amd import build as B

    try:
        B.hipcc()
        runtime = B.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build_host_sanitized(str(tmp_path))
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    # python and torch are not instrumented: no leak report at exit, and no report of
    # allocator pairs that cross their libraries
    env["ASAN_OPTIONS"] = "detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(root=ROOT, lib=lib, suite=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    res = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True,
                         timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "passed" in res.stdout and "failed" not in res.stdout, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
