"""The C ABI's host code under AddressSanitizer (CPU, no GPU needed).

Builds a second copy of libdflash2 whose host code (argument checks,
workspace layout, launch set-up) is instrumented with AddressSanitizer
(device code unchanged), then runs the ABI and host tests against it in a
child process with the clang runtime preloaded.  Every call those tests
make is validated and rejected (or is a no-op) before any launch, so the
whole of the host-side checking runs instrumented.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_abi_checks_clean_under_host_asan():
    from block_drafting_amd import build as B
    try:
        B.hipcc()
        runtime = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build(asan=True)
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               DFLASH2_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p",
                        "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py"),
                        os.path.join(ROOT, "tests", "test_host.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=900)
    assert "AddressSanitizer" not in r.stdout, r.stdout[-4000:]
    assert r.returncode == 0, r.stdout[-4000:]
    assert " passed" in r.stdout
