"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A second copy of libw2a8.so is built into a temporary folder with the host
pass instrumented (each sanitizer flag goes to the host compiler only; the
device code is compiled as usual and never runs here).  A C driver,
tests/asan/host_abi_check.c, built with the same sanitizers, then runs the
packers, the ternarizer, the size queries, the launch planner, the argument
validation and the tuning knobs (from several threads) on heap buffers of
exactly the documented sizes.  Any out-of-bounds access, leak or undefined
operation in the host code aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fno-omit-frame-pointer", "-g", "-O1"]


def _torch_lib():
    import torch
    return os.path.join(os.path.dirname(torch.__file__), "lib")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout[-4000:] + res.stderr[-4000:]
    return res


@pytest.mark.skipif(shutil.which("hipcc") is None or not os.path.exists(CLANG),
                    reason="needs hipcc and the ROCm clang")
def test_host_code_under_asan_and_ubsan(tmp_path):
    pkg = os.path.join(ROOT, "w2a8_gemv_amd")
    srcs = sorted(os.path.join(pkg, "csrc", f) for f in os.listdir(os.path.join(pkg, "csrc"))
                  if f.endswith(".hip"))
    tlib = _torch_lib()
    lib = str(tmp_path / "libw2a8_asan.so")
    _run(["hipcc", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared", *SAN,
          "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(pkg, "csrc"), *srcs,
          "-L", tlib, "-Wl,-rpath," + tlib, "-lamdhip64", "-o", lib])
    exe = str(tmp_path / "host_abi_check")
    _run([CLANG, *SAN, "-fsanitize=address,undefined", "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "asan", "host_abi_check.c"),
          "-L", str(tmp_path), "-lw2a8_asan", "-Wl,-rpath," + str(tmp_path),
          "-L", tlib, "-Wl,-rpath," + tlib, "-lamdhip64", "-lpthread", "-o", exe])
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""
    res = _run([exe], env=env, timeout=300)
    assert "host ABI checks passed" in res.stdout
