"""The C ABI tests again, against a build of the host layer (api.cpp) with
AddressSanitizer and UndefinedBehaviorSanitizer: every validation path,
workspace formula and error text runs with out-of-bounds, use-after-free,
overflow and invalid-value checks, and any report fails the run. CPU only (the
ABI tests launch nothing)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_under_host_sanitizers():
    from rank_compressed_kv_amd import build_sanitized as build
    lib = build.build()
    env = dict(os.environ)
    env.update(PALU_LIBRARY=lib, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, tail
