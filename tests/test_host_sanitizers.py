"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds the library with both sanitizers on its host code
(`build.build_sanitized`) and runs every ABI test that calls an entry point
against it in a child process with the ASan runtime preloaded.  The child must
pass and print no sanitizer report; any report aborts it
(halt_on_error / -fno-sanitize-recover).
"""
import os
import subprocess
import sys

import pytest

from sequence_length_latent_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_validation_under_host_asan_ubsan():
    runtime = b.sanitizer_runtime()
    if not os.path.exists(runtime):
        pytest.skip("ASan runtime not found next to the compiler")
    lib = b.build_sanitized(verbose=False)
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=66"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=67"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "_sanitized_abi.py"), lib],
                       env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
