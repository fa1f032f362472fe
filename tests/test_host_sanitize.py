"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): every csrc source built with host-side instrumentation, linked with
the driver tests/host_check/lla_host_check.cpp, which runs argument
validation, workspace and split planning over a grid of shapes, the
token-eviction page rule against its definition, eq. (4) scalars and the
thread-local error message from 8 threads.  No kernel is launched."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.timeout(600)
def test_host_code_under_asan_and_ubsan():
    sys.path.insert(0, os.path.join(HERE, "host_check"))
    import build_host_check  # imported here: the folder is not shipped to GPU runs
    exe = build_host_check.build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "host check OK" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
