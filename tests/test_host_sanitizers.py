"""The C ABI's host code (argument validation, workspace sizing and carving,
dispatch up to the first HIP call) under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed).

The library is rebuilt with the sanitizers on its host compilation only
(grouped_query_attention_gemv_amd.build --sanitize) and the host ABI tests
run against it in a child process with the sanitizer runtime preloaded; any
sanitizer report aborts that process.
"""
import os
import subprocess
import sys

from grouped_query_attention_gemv_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_tests_pass_under_asan_and_ubsan():
    lib = B.build(sanitize=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=B.asan_runtime(), GQA_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
