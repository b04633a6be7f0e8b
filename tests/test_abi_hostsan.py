"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The argument checks, the plans and the tile table (mhc_api.cpp,
mhc_tile_table.cpp) are rebuilt with both sanitizers on the host side only and
linked with the kernels' objects of the last in-tree build; test_abi.py's
checks that launch nothing (status strings, argument validation, plans, sizes
near the integer limits) then run in a child process that loads that build
with the sanitizer runtime preloaded. Any report (out-of-bounds access,
use-after-free, signed overflow, invalid enum or shift) ends the child with an
error and fails this test.
"""

import os
import subprocess
import sys

import pytest

from mhc_hyper_connection_pre_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _kernel_objects_present():
    return all(os.path.exists(os.path.join(B.OBJDIR, os.path.splitext(s)[0] + ".o"))
               for s in B.SOURCES if not s.endswith(".cpp"))


def test_abi_checks_under_host_sanitizers(tmp_path):
    if not _kernel_objects_present():
        pytest.skip("the in-tree build's objects are missing (run the build first)")
    runtime = B.sanitizer_runtime()
    if not runtime or not os.path.exists(runtime):
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    lib = B.build_hostsan_library()
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, MHC_ABI_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider", "-k", "validation or status or plan or integer_limits"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout and "skipped" not in r.stdout, r.stdout[-2000:]
