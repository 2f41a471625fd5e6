"""The library's host C++ (packer, planners, cache directory) under address
and undefined-behaviour sanitizers: tests/host/fuzz_host.cpp drives random
valid and invalid inputs through the C ABI, built with g++ from the same
sources as the library (no device code involved).  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunked_linear_attention_packed_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "fuzz_host")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host", "fuzz_host.cpp"),
           os.path.join(CSRC, "pack.cpp"), os.path.join(CSRC, "cache.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in (build.stderr or "").lower():
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert run.returncode == 0, run.stdout + run.stderr
    assert "host fuzz: ok" in run.stdout
