"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built with gcc/g++ and run: the C oracle driven through
every entry point (tests/host_sanitize/oracle_checks.c), and the C ABI's
host validation, abi.cpp, driven with ordinary, extreme and garbage
arguments (tests/host_sanitize/abi_checks.cpp).  No device code is compiled:
abi.cpp is the host-only part of the library.  Any sanitizer report aborts
the program and fails the test.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ROCM_INCLUDE = "/opt/rocm/include"


def _compiler(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not available")
    return path


def _build_and_run(cmd, exe, env_extra=None):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr and "unrecognized" in r.stderr:
        pytest.skip("compiler without sanitizer support")
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ)
    env.update({"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"})
    env.update(env_extra or {})
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    return r.stdout


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = _compiler("gcc")
    exe = str(tmp_path / "oracle_checks")
    cmd = [gcc, "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN,
           os.path.join(ROOT, "oracle", "moe_oracle.c"), os.path.join(HERE, "host_sanitize", "oracle_checks.c"),
           "-lm", "-o", exe]
    assert "oracle checks ok" in _build_and_run(cmd, exe, {"OMP_NUM_THREADS": "2"})


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    gxx = _compiler("g++")
    if not os.path.exists(os.path.join(ROCM_INCLUDE, "hip", "hip_runtime_api.h")):
        pytest.skip("HIP headers not available")
    csrc = os.path.join(ROOT, "quantized_expert_gemv_moe_amd", "csrc")
    exe = str(tmp_path / "abi_checks")
    cmd = [gxx, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(csrc, "abi.cpp"), os.path.join(HERE, "host_sanitize", "abi_checks.cpp"), "-o", exe]
    assert "abi checks ok" in _build_and_run(cmd, exe)
