"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): a copy of libdflash.so whose api.hip host side is instrumented
(device code unchanged) runs the CPU boundary and binding tests in a child
process with the sanitizer runtime preloaded. Covered: config guards and
create/destroy, state and workspace layouts of every config, binding and
argument validation of every entry point (each refused before any launch),
the error string, the block policy functions."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_is_clean_under_asan_and_ubsan():
    from block_diffusion_drafter_tap_amd import build as B
    try:
        lib = B.build_host_sanitized()
        rt = B.asan_runtime()
    except RuntimeError as e:       # no hipcc / sanitizer runtime in this environment
        pytest.skip(str(e))
    env = dict(os.environ, DFLASH_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_boundary.py", "tests/test_binding_checks.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
