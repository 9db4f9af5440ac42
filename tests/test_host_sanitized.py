"""The library's host code (argument checks, split plan, workspace layout,
the other entry points' checks) built for the CPU with AddressSanitizer and
UBSan against stand-ins for the HIP runtime and the kernel launchers, then
driven through its C entry points.  The stand-in launchers write every byte
of each workspace region the plan hands the kernels, so a layout that runs
past the size mla_decode_workspace_size returned shows up as a heap
overflow.  Compiled with g++ (host code only; no GPU code is built)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path_factory.mktemp("asan") / "host_checks")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "decode_attention_absorbed_amd", "csrc", "mla_api.cpp"),
           os.path.join(HERE, "hip_stubs.cpp"), os.path.join(HERE, "host_checks_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def test_host_code_under_asan_and_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([driver], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout[-2000:])
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-6000:])
    assert "ALL OK" in r.stdout
