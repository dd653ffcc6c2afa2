"""Build the oracle's shared library with gcc (plain C, no intrinsics, no HIP).

-ffp-contract=off keeps every fp32 multiply and divide separately rounded;
-fno-fast-math keeps IEEE semantics.  The oracle is test infrastructure.
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    src = os.path.join(_HERE, "oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
