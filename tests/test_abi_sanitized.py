"""The C ABI layer's host code under AddressSanitizer and UndefinedBehaviorSanitizer: hs_api.hip
rebuilt with both sanitizers on its host side (device code unchanged) and every CPU ABI test
(argument checks, planning, workspace sizing, the error paths) run against it in a subprocess
with the ASan runtime preloaded.  No GPU is touched: every call there fails validation first."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_clean_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from long_context_split_amd import build
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in this toolchain")
    lib = build.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, HYSPARSE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
