"""The library's host code (argument checks, problem geometry, workspace
layout, launch set-up, the reblock host calls) under AddressSanitizer and
UndefinedBehaviorSanitizer: a build with both sanitizers on the host pass
runs the C-ABI tests in a child process with the sanitizer runtime preloaded;
any report aborts that process.  CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

from block_sparse_attention_25_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_host_sanitizers(tmp_path):
    runtime = B.asan_runtime()
    if runtime is None or not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc or the AddressSanitizer runtime is not installed")
    lib = B.build_sanitized(str(tmp_path / "libbsa_sanitized.so"))
    # the host code really is instrumented: it calls the sanitizers' report hooks
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, BSA_LIBRARY=lib, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi.py")]
    res = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
