"""The host layer of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): tests/host_check_build.py compiles
api.hip's host side with both sanitizers and links it with the kernel
objects and tests/abi_host_check.c, whose checks cover argument validation,
ragged and grouped-key shapes, non-finite scales, the workspace queries and
the launch plans.  A sanitizer report or a failed check fails the test."""
import os
import sys

import pytest


@pytest.mark.timeout(900)
def test_host_layer_clean_under_asan_and_ubsan():
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import host_check_build
    host_check_build.build()
    p = host_check_build.run()
    assert p.returncode == 0, p.stdout[-4000:]
    assert "abi host checks passed" in p.stdout
    assert "ERROR: AddressSanitizer" not in p.stdout and "runtime error:" not in p.stdout
