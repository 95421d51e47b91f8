"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): sv_api.cpp built with g++ and linked against stub launchers
(tests/host_asan_driver.cpp), then every refusal path and a passing call of
each entry point, on exactly sized host buffers."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "adaptive_draft_verification_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_host_side_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = tmp_path / "host_checks"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", os.path.join(ROCM, "include"),
           os.path.join(CSRC, "sv_api.cpp"), os.path.join(HERE, "host_asan_driver.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1",
               LD_LIBRARY_PATH=os.path.join(ROCM, "lib") + ":" + os.environ.get("LD_LIBRARY_PATH", ""))
    env.pop("SV_DEBUG_CHECKS", None)
    env.pop("SV_FORCE_SYNC", None)
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "host checks passed" in run.stdout
