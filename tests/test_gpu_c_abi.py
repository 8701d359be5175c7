"""The library driven from a plain host program through its C ABI (no Python
binding, no PyTorch): closed-form checks of the indexer, both attention entry
points (unsplit and split + merged) and the merge. The program is built by
__graft_entry__.build() (tests/c_abi_build.py)."""
import os
import subprocess

import pytest

from c_abi_build import EXE

pytestmark = pytest.mark.gpu


def test_c_abi_closed_forms():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build() first")
    print("c-abi closed forms", flush=True)
    r = subprocess.run([EXE], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout
    assert r.stdout.strip().endswith("c-abi closed forms ok")
    assert "FAIL" not in r.stdout
