"""The library's host code (C ABI, argument validation, layer composition,
streamer, kernel launchers) built with AddressSanitizer, and the ABI tests run
against that build in a child process with the sanitizer runtime preloaded.
Device code is built as usual; no kernel is launched (the ABI tests need no
GPU)."""
import os
import subprocess
import sys

import pytest

from layer_streamed_frozen_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_tests_are_clean_under_host_asan():
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime under /opt/rocm/llvm")
    lib = build.build(asan=True)
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in out  # the host code really is instrumented
    env = dict(os.environ, LSF_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr
