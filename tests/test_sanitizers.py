"""The oracle and the C ABI's host code built with AddressSanitizer and UndefinedBehaviorSanitizer
and driven on the CPU (no GPU: HIP runtime calls and kernel launchers are host stubs).

tests/sanitize/driver.cpp calls every entry point with valid and rejected arguments (error codes,
workspace plans, the 32-bit offset limits, launch markers) and the oracle's functions on small
inputs and edge cases; any sanitizer finding aborts the program, and any unmet expectation makes
it exit non-zero.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc and g++")
def test_abi_host_code_and_oracle_under_asan_ubsan(tmp_path):
    inc = ["-I", os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include"),
           "-D__HIP_PLATFORM_AMD__"]
    csrc = os.path.join(ROOT, "diffusion_self_conditioning_amd", "csrc")
    objs = []
    for src, cc, extra in [
            (os.path.join(ROOT, "oracle", "softembed_oracle.c"), "gcc",
             ["-std=c11", "-fopenmp", "-ffp-contract=off"]),
            (os.path.join(csrc, "api.cpp"), "g++", ["-std=c++17"] + inc),
            (os.path.join(ROOT, "tests", "sanitize", "hip_stubs.cpp"), "g++", ["-std=c++17"] + inc),
            (os.path.join(ROOT, "tests", "sanitize", "driver.cpp"), "g++", ["-std=c++17"])]:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([cc, *SAN, *extra, "-c", src, "-o", obj], check=True)
        objs.append(obj)
    exe = str(tmp_path / "sanitized_driver")
    subprocess.run(["g++", *SAN, "-static-libasan", *objs, "-fopenmp", "-lm", "-o", exe],
                   check=True)
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out
    assert "OK: 0 failed expectations" in out, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
