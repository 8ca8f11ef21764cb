"""The C-ABI host validation (csrc/qmm_api.cpp) built for the CPU with
AddressSanitizer and driven through every error path and kernel selection
(tests/host_asan_driver.cpp, the HIP launchers stubbed out): an out-of-bounds
read or write, a use after free or a leak in the host code fails the test.
CPU only: g++ compiles the file against the ROCm headers; no GPU is touched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_weight_quantized_amd", "csrc")


@pytest.mark.slow
def test_host_validation_under_asan(tmp_path):
    gxx = shutil.which("g++")
    inc = "/opt/rocm/include"
    if not gxx or not os.path.isdir(inc):
        pytest.skip("g++ or the ROCm headers are not available")
    exe = tmp_path / "abi_asan"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", f"-I{inc}",
           os.path.join(CSRC, "qmm_api.cpp"), os.path.join(ROOT, "tests", "host_asan_driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "host validation ok" in r.stdout
