"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed).

The sanitized build of libfp8mla.so (host code of the C ABI instrumented,
every finding fatal; device code as in the release build) is loaded in a
child process that preloads the sanitizer runtime and runs every test of
test_abi.py against it: the argument checks, the status strings, the size
bounds of the extend call and the workspace queries all run instrumented.  A
memory error or undefined behaviour on any of those paths aborts the child.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

build = pytest.importorskip("fp8_paged_mla_amd.build")


def test_abi_host_code_under_sanitizers():
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("no hipcc")
    runtime = build.sanitizer_runtime()
    if not runtime:
        pytest.skip("no shared AddressSanitizer runtime in this toolchain")
    lib = build.build_sanitized()
    # the library really is instrumented: it calls into the sanitizer runtime
    nm = shutil.which("nm")
    if nm:
        syms = subprocess.run([nm, "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_" in syms and "__ubsan_handle_" in syms
    env = dict(os.environ)
    env.update({
        "FP8MLA_TEST_LIB": lib,
        "LD_PRELOAD": runtime,
        # Python and torch are not instrumented and keep memory until exit
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, out
    assert " passed" in r.stdout, out
