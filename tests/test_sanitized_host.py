"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
the host-side tests (argument validation, capacity and workspace sizes,
stage choice, operand spans, the binding's checks, the dispatch check) run in
a child process that preloads the sanitizer runtime and loads the sanitized
build.  Any sanitizer report aborts the child (UBSan is built without
recovery) and fails this test.  The sanitized build is kept in _build/san and
redone only when a source changed."""
import os
import subprocess
import sys

from top_routing_dispatch_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_abi_host.py", "tests/test_debug_checks.py"]


def test_host_code_clean_under_asan_and_ubsan():
    lib = B.build_sanitized()
    env = dict(os.environ)
    env.update(LD_PRELOAD=B.sanitizer_runtime(), MOE_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", *HOST_TESTS, "-q", "-x", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    tail = "\n".join(r.stdout.splitlines()[-40:])
    assert r.returncode == 0, f"sanitized host tests failed ({r.returncode}):\n{tail}"
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error:" not in r.stdout, tail
    assert " passed" in r.stdout, tail
