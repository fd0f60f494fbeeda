"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

api.cpp and plan.cpp are compiled with the sanitizers on their host side,
linked with launchers that stand in for the kernels (tests/host_sanitize/
stub_launch.cpp: each reports "no device") and driven by a C program that
makes every exported call with invalid, overflowing, overlapping and valid
arguments (tests/host_sanitize/driver.c). No GPU is used and no device
pointer is dereferenced.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_linear_recurrent_amd", "csrc")
INC = os.path.join(ROOT, "include")
HERE = os.path.join(ROOT, "tests", "host_sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}"
    return r


@pytest.mark.timeout(600)
def test_abi_host_code_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("the ROCm compilers are not installed")
    san_host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", INC, "-I", CSRC]
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"), os.path.join(HERE, "stub_launch.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *flags, *san_host, "-x", "hip", "-c", src, "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "driver.o")
    _run([CLANG, "-O1", "-g", "-std=c99", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", INC, "-c", os.path.join(HERE, "driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_sanitize")
    _run([CLANGXX, "-fsanitize=address,undefined", *objs, drv, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=300)
    assert "ERROR: AddressSanitizer" not in r.stdout, r.stdout[-4000:]
    assert "runtime error" not in r.stdout, r.stdout[-4000:]
    assert r.returncode == 0, r.stdout[-4000:]
    assert " 0 failures" in r.stdout, r.stdout[-4000:]
