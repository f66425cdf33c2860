"""The host code built with AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, gcc/g++): the binary64 oracle driven over every path by
tests/sanitize/oracle_driver.c, and the C ABI's admission, argument checks,
launch sequencing and chunk planning (csrc/sa_api.cpp and the planning helpers
of csrc/sa_internal.h) driven by tests/sanitize/api_driver.cpp against
host-only launcher stand-ins.  Any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "causal_streaming_attention_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=ENV)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", *SAN, "-fopenmp",
                    os.path.join(ROOT, "oracle", "sa_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
                    "-o", exe, "-lm"], check=True)
    assert "oracle-sanitize: ok" in _run(exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"),
                    reason="g++ or the HIP headers not installed")
def test_abi_host_code_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "api_san")
    inc = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    subprocess.run(["g++", "-std=c++17", "-Wall", *SAN, *inc, os.path.join(CSRC, "sa_api.cpp"),
                    os.path.join(HERE, "api_stubs.cpp"), os.path.join(HERE, "api_driver.cpp"), "-o", exe],
                   check=True)
    assert "api-sanitize: ok" in _run(exe)
