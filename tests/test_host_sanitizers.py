"""The C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

kvq_api.cpp (argument validation, page-table and workspace sizes, the
workspace layout) is rebuilt with g++ -fsanitize=address,undefined and linked
with the device objects of the regular build; the ABI tests then run against
that library in a child process with gcc's ASan runtime preloaded.  Any
out-of-bounds access, use after free or undefined behaviour on those paths
aborts the child, which fails this test.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        return None
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_abi_checks_under_host_sanitizers():
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    from rotated_int2_kv_centering_amd import build

    lib = build.build_host_sanitized()
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, KVQ_TEST_LIB=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1")
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                           os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=900)
    tail = (proc.stdout + proc.stderr)[-4000:]
    assert proc.returncode == 0, tail
    assert "passed" in proc.stdout and "AddressSanitizer" not in proc.stderr and "runtime error" not in proc.stderr, tail
