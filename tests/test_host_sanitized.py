"""The C-ABI layer (argument validation, workspace carving, launch sequences of every entry point)
built with the host compiler under AddressSanitizer and UndefinedBehaviorSanitizer and driven
without a GPU: the kernel launchers and the HIP runtime calls are host stand-ins
(tests/host_abi/stubs.cpp) that check every buffer a launch would touch against the buffers the
driver (tests/host_abi/driver.cpp) registered, at the tiny and the full 40-layer sizes, in bf16 and
fp32, with the variants, state rows and MXFP8 / MXFP4 precisions."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_c_abi_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "host_abi")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "world_action_video_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "host_abi", "stubs.cpp"),
           os.path.join(ROOT, "tests", "host_abi", "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    # verify_asan_link_order=0: the sanitizer runtime need not be first among the preloaded libraries
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host_abi: OK" in r.stdout
