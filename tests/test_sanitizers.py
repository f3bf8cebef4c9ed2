"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the host-side code,
without a GPU: the C ABI's argument validation (api.cpp, built with g++ with
the kernel launchers replaced by aborting stubs, so no path may reach a
launch) and the fp64 oracle (oracle.c with OpenMP, every function on small odd
shapes and on each codec's special values).  Any invalid memory access,
leak in the oracle or undefined operation fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_api_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_api_checks")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "state_space_recurrence_amd", "csrc"),
          os.path.join(ROOT, "state_space_recurrence_amd", "csrc", "api.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "host_api_checks.cpp"),
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # the HIP runtime's own allocations are not this code's to check for leaks
    out = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1"})
    assert "0 failed" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"),
          "-lm", "-o", exe])
    out = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1"})
    assert "oracle sanitizer run" in out
