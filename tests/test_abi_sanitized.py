"""The host side of the C ABI (descriptor and pointer validation, workspace
layout, the no-allocation entry point's size check) under AddressSanitizer and
UndefinedBehaviorSanitizer: a copy of the library whose host code is
instrumented (device code unchanged) runs the host-only ABI tests in a child
process with the sanitizer runtime preloaded.  Any sanitizer report aborts the
child and fails this test.  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_code_under_asan_ubsan():
    from chunk_weight_rnn_amd import build
    try:
        runtime = build.sanitizer_runtime()
        build.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build_sanitized()
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True)
    assert "__asan_report" in nm.stdout and "__ubsan_handle" in nm.stdout, "host code is not instrumented"
    env = dict(os.environ, E2TTT_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_zz_no_alloc.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in r.stdout, tail
