"""Build the C-ABI closed-form check (tests/c_abi_closed_forms.cpp): a host
program that links the in-tree libsa.so and calls only HIP runtime functions
and the sa_* entry points. Built by __graft_entry__.build(); run by
tests/test_gpu_c_abi.py."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_closed_forms.cpp")
EXE = os.path.join(HERE, "c_abi_closed_forms")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "sparse_block_indexed_amd")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"), SRC, "-o", EXE,
           "-L", pkg, "-lsa", "-Wl,-rpath,$ORIGIN/../sparse_block_indexed_amd"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
