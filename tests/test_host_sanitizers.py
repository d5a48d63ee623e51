"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

* tests/sanitize/host_checks.cpp drives the library's csrc/plan.cpp (plan
  geometry, argument checks, error strings) through 1,500 random plans and
  every plan error path, built with g++ for the host only (no HIP code, no
  GPU);
* tests/sanitize/oracle_checks.c drives the oracle's C code on buffers of
  exactly the sizes its contract names (3,000 random cases, every element
  type, pack then all-gather back).

Each must finish without a sanitizer report and with every expected result.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "parameter_layout_collectives_amd", "csrc", "plan.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp")]
ROCM_INCLUDE = "/opt/rocm/include"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _run(exe, marker):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    if run.returncode != 0 and "LeakSanitizer has encountered a fatal error" in run.stderr:
        # the leak checker itself cannot run here (e.g. under ptrace): keep
        # the address and undefined-behaviour checks
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
        run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-6000:])
    assert marker in run.stdout
    assert "runtime error" not in run.stderr and "ERROR: AddressSanitizer" not in run.stderr


def test_host_code_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "host_checks")
    build = subprocess.run(
        [gxx, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, *SAN, *SOURCES,
         "-o", exe],
        capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    _run(exe, "host checks passed")


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("needs gcc")
    exe = str(tmp_path / "oracle_checks")
    build = subprocess.run(
        [gcc, "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", *SAN,
         os.path.join(ROOT, "oracle", "oracle.c"),
         os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"), "-o", exe, "-lm"],
        capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    _run(exe, "oracle checks passed")
