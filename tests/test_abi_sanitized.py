"""The C ABI layer (csrc/api.cpp) built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer and driven through every entry point's validation
and accepted paths (tests/abi_sanitize.cpp: stub HIP device queries, stand-in
launchers that check what reaches them). Sizes near INT64_MAX are included, so
an overflowing size product in a check fails here as a sanitizer report."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_abi_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "fp8_fine_grained_fp8bq_amd", "csrc"),
           os.path.join(ROOT, "fp8_fine_grained_fp8bq_amd", "csrc", "api.cpp"),
           os.path.join(HERE, "abi_sanitize.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower() and "cannot find" in build.stderr.lower():
        pytest.skip("sanitizer runtimes not installed: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    print(res.stdout, res.stderr[-3000:])
    assert res.returncode == 0, res.stdout + res.stderr[-3000:]
    assert "0 failed checks" in res.stdout
