"""Host-code sanitizers, on the CPU: the C ABI's validation and dispatch
(api.hip built as plain C++ with stub launchers) and the float64 oracle, each
built with AddressSanitizer and UndefinedBehaviorSanitizer (errors abort) and
run on a driver that exercises every entry point.  The GPU kernels are not
built here; these builds cover host code only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _build_and_run(cmd, exe, tmp_path):
    if shutil.which(cmd[0]) is None:
        pytest.skip(f"{cmd[0]} not available")
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp_path)
    assert r.returncode == 0, f"build failed:\n{r.stdout}\n{r.stderr}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"sanitized run failed:\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-x", "c++",
           os.path.join(ROOT, "delta_rule_recurrent_chunkwise_amd", "csrc", "api.hip"), "-x", "none",
           os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", exe]
    out = _build_and_run(cmd, exe, tmp_path)
    assert "no sanitizer report" in out


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-std=c11", *SAN, "-fopenmp", os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"]
    out = _build_and_run(cmd, exe, tmp_path)
    assert "no sanitizer report" in out
