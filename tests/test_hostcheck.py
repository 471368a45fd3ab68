"""The C ABI's host-side argument validation, compiled for the CPU alone with
AddressSanitizer and UndefinedBehaviorSanitizer (g++) and linked against
stand-in launchers that record what would have been launched
(tests/hostcheck/host_validation_check.cpp).  Every argument error of
tests/test_abi.py is returned with nothing launched, and the accepted calls
hand the kernels the right arguments, with no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_validation_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.fail("g++ is needed to build the host-validation check")
    exe = str(tmp_path / "hostcheck")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "diffusion_transformer_joint_token_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "hostcheck", "host_validation_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    # verify_asan_link_order=0: the environment may preload other libraries
    # ahead of the sanitizer runtime.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "cases passed" in run.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
