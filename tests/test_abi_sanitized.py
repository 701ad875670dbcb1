"""The C API's host code (argument checks, workspace queries, status strings,
kernel selection) built with AddressSanitizer and UndefinedBehaviorSanitizer,
with host stubs for its device-side functions, runs the ABI tests of
test_abi.py: any memory or undefined-behaviour error aborts the run. Host
only (the build uses the host compiler; nothing is launched)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

BOOT = """
import sys
import causal_self_exchange_amd.relation as R
R.LIB_PATH = sys.argv[1]
import pytest
sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider', sys.argv[2]]))
"""


@pytest.mark.timeout(600)
def test_abi_tests_pass_under_host_sanitizers(tmp_path):
    if shutil.which(os.environ.get("CXX_HOST", "g++")) is None:
        pytest.skip("no host C++ compiler")
    from causal_self_exchange_amd.sanitize import build_host
    lib = build_host.build(str(tmp_path))
    env = dict(os.environ)
    # The sanitizer runtimes are loaded as the library's dependencies.
    env["ASAN_OPTIONS"] = "verify_asan_link_order=0:detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", BOOT, lib, os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=550)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
