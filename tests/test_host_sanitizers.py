"""The host library (quantizers, bitstreams, device layouts) under AddressSanitizer and
UndefinedBehaviorSanitizer: host.cpp built alone by g++ with both sanitizers (aborting on the
first report), and the host tests run against it in a child process that preloads the ASan
runtime. CPU only; skipped where g++ or its ASan runtime is missing."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    gxx = shutil.which("g++")
    if not gxx:
        return None
    path = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_tests_pass_under_asan_and_ubsan():
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("g++ with an ASan runtime is not available")
    sys.path.insert(0, os.path.join(ROOT, "dequant_gemv_q4g32_amd"))
    try:
        import build as qg_build
    finally:
        sys.path.pop(0)
    lib = qg_build.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=asan, QGEMV_HOST_ONLY_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:xdist", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_host_library.py"),
                          os.path.join(ROOT, "tests", "test_host_fuzz.py"),
                          "-k", "not entry_point and not exports_every"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
