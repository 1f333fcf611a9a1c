"""The C ABI layer (csrc/sia_api.cpp: validation, workspace layout, dispatch)
built for the host with AddressSanitizer and UndefinedBehaviorSanitizer and
driven through every entry point's accepted and rejected argument paths
(tests/asan/abi_driver.cpp).  Kernel launchers and the HIP runtime queries are
host stubs (tests/asan/stubs.cpp) that count launches: a rejected call must
return its documented status and launch nothing.  No GPU is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "asan")


def test_abi_layer_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / "abi_asan")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "sparse_index_attention_amd", "csrc", "sia_api.cpp"), os.path.join(HERE, "stubs.cpp"),
           os.path.join(HERE, "abi_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "abi driver ok" in r.stdout
