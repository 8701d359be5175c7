"""Build libsa.so in-tree with hipcc for gfx950 (cross-compiles without a GPU)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsa.so")
SOURCES = ["sa_api.cpp", "sa_attention.hip", "sa_indexer.hip", "sa_merge.hip", "sa_noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          # packed fp32 instructions stay off (hipcc's host pass warns it does not know the feature)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# keep MFMA accumulators in ordinary VGPRs (device compilation only)
DEVICE_ONLY = ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "argument unused during compilation" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every source and link libsa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmd = [HIPCC] + COMMON + ["-I", os.path.join(HERE, "..", "include")]
        if src.endswith(".hip"):
            cmd += DEVICE_ONLY
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
