"""The C-ABI layer and split planner (pdllm_abi.cpp, plan.cpp) built for the
host alone with AddressSanitizer and UndefinedBehaviorSanitizer, linked with
stub kernel launchers (tests/hostcheck/stub_launchers.cpp), and driven through
every entry point's validation paths and a planner sweep
(tests/hostcheck/abi_hostcheck.cpp).  A sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "diffusion_long_context_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "hostcheck")


def test_abi_and_planner_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("g++ and the HIP headers are needed for the host build")
    exe = str(tmp_path / "abi_hostcheck")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "pdllm_abi.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(HERE, "stub_launchers.cpp"), os.path.join(HERE, "abi_hostcheck.cpp"),
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    assert "0 failure(s)" in run.stdout
