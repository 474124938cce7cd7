"""The host C++ of the library (block manager with its prefix cache, and the
scheduler: hand-linked free lists, a hash tree, refcounts) built alone with
AddressSanitizer and UndefinedBehaviorSanitizer, and its CPU tests run
against that build in a child process.  Any sanitizer finding aborts the
child, so the test passes only if every case runs clean."""

import os
import subprocess
import sys

import pytest

from tests import harness

HOST_TESTS = ["tests/test_block_manager.py", "tests/test_prefix_cache.py", "tests/test_scheduler.py"]


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_host_cpp_tests_pass_under_asan_and_ubsan():
    from paged_kv_cache_326_amd import build

    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no AddressSanitizer runtime for g++ here")
    lib = build.build_host_sanitized()
    env = dict(os.environ)
    env["PA_LIB"] = lib
    # The interpreter is not instrumented: the ASan runtime must come first.
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    # CPython keeps objects alive until exit by design; leak reports would
    # be about the interpreter, not the library.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *HOST_TESTS],
                       cwd=harness.ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and " failed" not in out, out[-2000:]
