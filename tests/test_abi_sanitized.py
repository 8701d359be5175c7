"""Every C-ABI entry point's host validation, run from a host program whose
C-ABI layer is built with AddressSanitizer and UndefinedBehaviorSanitizer
(tests/c_abi_validation.cpp, built by __graft_entry__.build()). No GPU: each
call is refused, or is a no-op, before any HIP call."""
import os
import subprocess

import pytest

from c_abi_build import VAL_EXE


def test_host_validation_under_address_and_undefined_behaviour_sanitizers():
    if not os.path.exists(VAL_EXE):
        pytest.fail(f"{VAL_EXE} is missing: run __graft_entry__.build() first")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([VAL_EXE], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout
    assert r.stdout.strip().endswith("c-abi validation ok"), r.stdout
    assert "runtime error" not in r.stdout and "AddressSanitizer" not in r.stdout, r.stdout
