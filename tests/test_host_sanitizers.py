"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers are built with the sanitizers and run:
  * tests/sanitize/api_driver.cpp with the C-ABI host code (gdn_api.cpp): every
    argument check, workspace layout and dispatch decision, the kernel
    launchers and HIP runtime calls replaced by stubs that touch every byte
    range a layout hands a kernel (an overrun is an ASan report);
  * tests/sanitize/oracle_driver.c with the C oracle.
A sanitizer report makes the driver exit non-zero; the test also fails on any
report text in its output."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def _require(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def test_api_host_code_under_sanitizers():
    _require("g++")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "api_driver")
    csrc = os.path.join(ROOT, "hybrid_linear_attention_delta_amd", "csrc")
    rc, log = _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"), os.path.join(csrc, "gdn_api.cpp"),
                    "-o", exe])
    assert rc == 0, log
    rc, log = _run([exe], env=ENV, timeout=300)
    print(log)
    assert rc == 0, log
    assert "ERROR: AddressSanitizer" not in log and "runtime error" not in log, log


def test_oracle_under_sanitizers():
    _require("gcc")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    rc, log = _run(["gcc", "-std=c11", *SAN, "-pthread", "-ffp-contract=off",
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm", "-o", exe])
    assert rc == 0, log
    rc, log = _run([exe], env=ENV, timeout=300)
    print(log)
    assert rc == 0, log
    assert "ERROR: AddressSanitizer" not in log and "runtime error" not in log, log
