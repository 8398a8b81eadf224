"""Host-only argument-validation test of the C ABI under sanitizers.

Builds tests/host/validation_test.cpp together with the real host dispatcher
and planning sources (csrc/adaln_api.cpp, csrc/adaln_plan.cpp) with the host
compiler, AddressSanitizer and UndefinedBehaviorSanitizer, and runs it.  The
kernel launchers and the device query are stubs inside the test file, so no
GPU and no HIP runtime library is needed; only the HIP runtime headers are.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "diffusion_transformer_adaln_amd", "csrc")
HIP_INCLUDE = "/opt/rocm/include"
SOURCES = [
    os.path.join(ROOT, "tests", "host", "validation_test.cpp"),
    os.path.join(CSRC, "adaln_api.cpp"),
    os.path.join(CSRC, "adaln_plan.cpp"),
]


def test_host_validation_sanitized(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isfile(os.path.join(HIP_INCLUDE, "hip", "hip_runtime_api.h")):
        pytest.skip("needs g++ and the HIP runtime headers")
    exe = str(tmp_path / "validation_test")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Werror",
           "-D__HIP_PLATFORM_AMD__", "-I" + HIP_INCLUDE, "-I" + os.path.join(ROOT, "include"),
           *SOURCES, "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert " 0 failures" in out, out[-4000:]
