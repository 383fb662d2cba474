"""The C ABI's argument checking under the address and undefined-behaviour sanitizers, on the CPU.

ram_api.cpp is built host-only with g++ (-fsanitize=address,undefined, no recovery), its kernel
launchers and HIP runtime calls stubbed (tests/sanitize/stub_hip.cpp), and linked with a driver
(tests/sanitize/abi_cases.cpp) that runs the same invalid-argument and empty-input cases as
test_abi.py. Any sanitizer report aborts the driver; any unexpected status is a failed case."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_san")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "ring_attention_merge_amd", "csrc", "ram_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "stub_hip.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "abi_cases.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout)
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    assert r.returncode == 0, r.stdout + r.stderr
    assert " cases as expected" in r.stdout
