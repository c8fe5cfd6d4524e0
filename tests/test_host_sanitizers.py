"""The host-side library code under AddressSanitizer and
UndefinedBehaviorSanitizer: the host C++ sources (argument checks,
parameter construction for every init entry point, polar codebooks) are
rebuilt with both sanitizers and the CPU library tests run against that
build in a child process with the sanitizer runtime preloaded.  Any report
aborts the child (halt_on_error), which fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_host_library_tests_pass_under_asan_and_ubsan():
    from vector_quantization_quantize_amd import _sanitize_build as sb
    rt = sb.runtime()
    if rt is None:
        pytest.skip("no shared ASan runtime next to hipcc")
    lib = sb.build()
    env = dict(os.environ)
    env.update({"LD_PRELOAD": rt, "TQ_LIBRARY": lib,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_lib_host.py"), "-q",
                          "-x", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "runtime error" not in tail and "AddressSanitizer" not in tail, tail
