"""Build the two host programs that drive libsa's C ABI directly (no Python):
- tests/c_abi_closed_forms.cpp links the in-tree libsa.so and checks closed-form
  results on the GPU (run by tests/test_gpu_c_abi.py);
- tests/c_abi_validation.cpp links the C-ABI layer compiled with
  AddressSanitizer and UndefinedBehaviorSanitizer on its host code and checks
  every entry point's host validation, with no GPU (run by
  tests/test_abi_sanitized.py).
Built by __graft_entry__.build()."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_closed_forms.cpp")
EXE = os.path.join(HERE, "c_abi_closed_forms")
VAL_SRC = os.path.join(HERE, "c_abi_validation.cpp")
VAL_EXE = os.path.join(HERE, "c_abi_validation_san")
OBJ = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")


def build(verbose: bool = False) -> str:
    """Both programs; the library (and its object files) must have been built first."""
    pkg = os.path.join(ROOT, "sparse_block_indexed_amd")
    inc = os.path.join(ROOT, "include")
    _run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall", "-I", inc, SRC, "-o", EXE,
          "-L", pkg, "-lsa", "-Wl,-rpath,$ORIGIN/../sparse_block_indexed_amd"], verbose)
    # host code only is sanitized (each sanitizer flag applies to the host pass)
    os.makedirs(OBJ, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    common = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer", "-I", inc]
    api_o = os.path.join(OBJ, "sa_api_san.o")
    val_o = os.path.join(OBJ, "c_abi_validation.o")
    _run(common + san + ["-c", os.path.join(pkg, "csrc", "sa_api.cpp"), "-o", api_o], verbose)
    _run(common + san + ["-c", VAL_SRC, "-o", val_o], verbose)
    kernels = [os.path.join(pkg, "_build", f + ".o")
               for f in ("sa_attention.hip", "sa_indexer.hip", "sa_merge.hip", "sa_noalloc.hip")]
    _run([HIPCC, "--offload-arch=gfx950", "-fno-gpu-sanitize", "-fsanitize=address", "-fsanitize=undefined", val_o, api_o] + kernels + ["-o", VAL_EXE], verbose)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
