"""The C-ABI argument checks built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer (no device code: the launchers are host stubs
that count calls) and driven through every entry point with rejected and
accepted arguments (CPU only)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM_INC = "/opt/rocm/include"

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INC),
                                reason="needs g++ and the HIP headers")


def test_abi_checks_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_sanitize")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INC,
           os.path.join(ROOT, "w4a4_post_quantized_channel_amd", "csrc", "abi.cpp"),
           os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "ok: 0 failures" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
