"""Build libw2a8.so in-tree with hipcc for gfx950.

The library links the HIP runtime that PyTorch ships (same soname as the
system one), with an rpath to it, so that a process that has imported torch
and then loads this library uses one HIP runtime and torch's stream handles
are valid here.

Flags:
  --offload-arch=gfx950   CDNA4 only; no other targets, no fallbacks
  -O3 -ffp-contract=off   fp32 epilogue / quantizer ops stay separately rounded
  -Xclang -target-feature -Xclang -packed-fp32-ops
                          no packed fp32 instructions (v_pk_*_f32)
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libw2a8.so")
# Measurement helper for bench.py (a pure streaming read), not the library.
READREF_PATH = os.path.join(PKG, "readref", "libw2a8_readref.so")


def _torch_lib_dir() -> str:
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        raise RuntimeError("PyTorch (ROCm build) is required to build libw2a8.so")
    return os.path.join(list(spec.submodule_search_locations)[0], "lib")


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _hipcc(srcs, out, verbose):
    tlib = _torch_lib_dir()
    tmp = out + ".tmp"
    cmd = [
        "hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
        *srcs,
        "-L", tlib, "-Wl,-rpath," + tlib, "-lamdhip64",
        "-o", tmp,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    errs = [l for l in res.stderr.splitlines()
            if l.strip() and "packed-fp32-ops" not in l]
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _hipcc(sources(), LIB_PATH, verbose)
    _hipcc([os.path.join(PKG, "readref", "stream_read.hip")], READREF_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
