"""The host code of the library (packers, bitwidth allocation, channel
order: csrc/pack.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.
g++ builds it with tests/host_sanitize.cpp, a driver that runs every host
entry point on several shapes and bitmaps and through its error paths; the
sanitizers abort on the first memory or undefined-behaviour error."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "gemm_block_bit_amd", "csrc"),
           os.path.join(ROOT, "tests", "host_sanitize.cpp"),
           os.path.join(ROOT, "gemm_block_bit_amd", "csrc", "pack.cpp"),
           "-pthread", "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    # the environment is passed on unchanged; ASan is told not to insist on
    # coming first among the loaded libraries
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "ok" in r.stdout
