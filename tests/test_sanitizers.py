"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer:

* the fp64 oracle (tests/sanitize/oracle_driver.c: every entry point on
  small problems of every cell, and bad arguments);
* the library's ABI layer (pararnn.cpp: argument validation and workspace
  planning), compiled for the host only with the sanitizers and linked with
  the product build's kernel objects; tests/sanitize/abi_driver.cpp drives
  every path that returns before a HIP call, so no GPU is needed.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
PKG = os.path.join(ROOT, "nonlinear_rnn_evaluation_newton_amd")
CSRC = os.path.join(PKG, "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def check_clean(r, tag):
    out = r.stdout + r.stderr
    assert tag + ": ok" in out, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    check_clean(subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300), "oracle driver")


@pytest.mark.skipif(not os.path.exists(CLANG), reason="needs the ROCm clang")
def test_abi_validation_under_sanitizers(tmp_path):
    from nonlinear_rnn_evaluation_newton_amd import build
    objdir = build.OBJDIR
    kernels = [os.path.join(objdir, os.path.basename(s) + ".o") for s in build.sources() if not s.endswith(".cpp")]
    if not all(os.path.exists(o) for o in kernels):
        build.build()
    abi = str(tmp_path / "pararnn_san.o")
    run([CLANG, "-x", "hip", "--offload-host-only", "--rocm-path=/opt/rocm", "-std=c++17", "-O1", "-g", "-fPIC",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Xarch_host", "-fsanitize=address", "-Xarch_host",
         "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all", "-Wno-unused-value", "-Wno-unused-result",
         "-c", os.path.join(CSRC, "pararnn.cpp"), "-o", abi])
    drv = str(tmp_path / "abi_driver.o")
    run(["g++", "-std=c++17", "-O1", "-g", "-I", os.path.join(ROOT, "include"), "-fsanitize=address,undefined",
         "-c", os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    run([CLANG, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", drv, abi] + kernels +
        ["-o", exe, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    check_clean(subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300), "abi driver")
