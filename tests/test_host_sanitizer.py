"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer.

build() also makes a host-check library: api.cpp (argument validation,
workspace sizing, dispatch) compiled by g++ with both sanitizers, linked with
the release kernel objects.  This runs the boundary tests (tests/test_boundary.py:
every exported symbol, every rejected argument, the workspace queries) in a
child process against that library, with the sanitizer runtime preloaded;
any report aborts the child and fails here.  CPU only: the rejected calls
return before anything reaches the HIP runtime.
"""
import os
import subprocess
import sys

import pytest

from grouped_gemm_moe_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_boundary_under_host_sanitizers():
    if not os.path.exists(B.HOST_CHECK_LIB):
        pytest.skip("host-check library not built (build() makes it)")
    env = B.host_check_env()
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=600)
    assert p.returncode == 0, p.stdout[-4000:]
    assert "passed" in p.stdout and "ERROR: AddressSanitizer" not in p.stdout, p.stdout[-4000:]
    assert "runtime error" not in p.stdout, p.stdout[-4000:]
