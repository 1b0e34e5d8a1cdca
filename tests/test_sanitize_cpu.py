"""The C-ABI layer (csrc/api.cpp) and the slicing planner (csrc/slicing.cpp)
built for the CPU with AddressSanitizer and UndefinedBehaviorSanitizer,
with the kernel launchers replaced by range-checking stand-ins
(tests/sanitize/stubs.cpp), and driven through every entry point
(tests/sanitize/driver.cpp): no memory error, no undefined behaviour, every
status as expected, and every buffer region a launch would address inside
the caller's buffers."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "token_transformer_layer_amd", "csrc")
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_abi_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "sanitize", "driver.cpp"), os.path.join(ROOT, "tests", "sanitize", "stubs.cpp"),
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "slicing.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "sanitize ok" in run.stdout
