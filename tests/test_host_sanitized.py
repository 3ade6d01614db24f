"""The library's host code (argument validation, the host packer, planning
and workspace sizing) under AddressSanitizer and UndefinedBehaviorSanitizer.

A host-only build (no device code: nothing here launches a kernel) runs the
CPU ABI tests in a subprocess with the sanitizer runtime preloaded; a
sanitizer report ends that process with its own exit code and fails this
test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")


def test_abi_suite_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    import tree_verify_amd.build as B
    try:
        rt = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build_host_sanitized(str(tmp_path))
    code = ("import sys; sys.path[:0] = [%r, %r]; import tree_verify_amd as tv; tv.LIB_PATH = %r; "
            "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))"
            % (ROOT, TESTS, lib, os.path.join(TESTS, "test_abi.py")))
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail
