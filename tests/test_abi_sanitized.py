"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): tests/native/abi_hostcheck.cpp links api.cpp and gemm_plan.cpp
with stub launchers, built with g++ -fsanitize=address,undefined, and drives
the validation paths and the host plans with exact-size host buffers. Any
sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "invariant_bi_mm_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_hostcheck")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "gemm_plan.cpp"),
           os.path.join(ROOT, "tests", "native", "abi_hostcheck.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failures" in r.stdout
