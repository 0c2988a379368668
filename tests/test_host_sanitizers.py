"""The host-side ABI tests (tests/test_abi_host.py) run against a build of the
library whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer
(gated_linear_attention_chunked_amd/build_sanitize.py), in a child process with
the sanitizer runtime preloaded: every argument check of the C ABI, on valid and
invalid arguments, must run without a memory or undefined-behaviour report.
No GPU is needed (every case stops in the host checks)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_abi_host_checks_under_asan_and_ubsan():
    from gated_linear_attention_chunked_amd import build_sanitize
    rt = build_sanitize.runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this ROCm install")
    lib = build_sanitize.build()
    env = dict(os.environ, LIZARD_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: a sanitizer report goes to the child's stderr, not to pytest's capture
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, out[-3000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out
    assert " passed" in r.stdout
