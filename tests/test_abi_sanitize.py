"""The C ABI's host-side argument checks (csrc/api.cpp) under the host compiler's address
and undefined-behaviour sanitizers: built against stub launchers (no HIP, no GPU) and
driven with 200,000 seeded sets of valid, edge and random arguments
(tests/host_sanitize/abi_fuzz.cpp).  Any overflow or out-of-bounds access aborts it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_clean_under_asan_and_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "abi_fuzz"
    srcs = [os.path.join(ROOT, "paged_gqa_decode_kv_amd", "csrc", "api.cpp"),
            os.path.join(ROOT, "tests", "host_sanitize", "stub_launch.cpp"),
            os.path.join(ROOT, "tests", "host_sanitize", "abi_fuzz.cpp")]
    build = subprocess.run([cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                            "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                            *srcs, "-o", str(exe)], capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr and "cannot find" in build.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "calls accepted" in run.stdout
