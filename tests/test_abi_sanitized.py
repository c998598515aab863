"""The ABI validation tests (tests/test_abi.py) against a build of the host
library with AddressSanitizer and UndefinedBehaviorSanitizer on its host
code: every rejected call, status code and message path runs under the
sanitizers.  CPU only; builds into _build/sanitized."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_validation_paths_are_clean_under_asan_and_ubsan():
    from block_diffusion_drafting_dflash_amd import build
    lib = build.build_sanitized(os.path.join(ROOT, "_build", "sanitized"))
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib],
                          capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    env.update({
        "DFLASH_LIB": lib,
        "LD_PRELOAD": build.asan_runtime(),
        # the interpreter itself is not instrumented: its allocations are
        # not leak-checked; any report in the library is fatal
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p",
                        "no:cacheprovider", os.path.join(ROOT, "tests",
                                                         "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    # the sanitized build is the one that was loaded
    assert "passed" in r.stdout
