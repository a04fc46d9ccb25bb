"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/host_driver.cpp is compiled with g++ together with
rc_host.cpp (the library's only host source), with the kernel launchers
replaced by counting stubs, so no GPU and no HIP runtime are involved.  It
runs hand-picked rejections of every entry point, a valid call sequence,
injected launch failures and a seeded fuzz over ring fields and arguments;
any sanitizer report makes the run fail.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "autoregressive_video_diffusion_ring_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_host_code_under_asan_and_ubsan():
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "host_driver_asan")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "rc_host.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(run.stdout[-2000:])
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "0 failures" in run.stdout and run.stdout.strip().endswith("ok")
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
