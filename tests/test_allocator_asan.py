"""The block allocator under the address and undefined-behaviour sanitizers:
tests/native/allocator_stress.cpp and csrc/allocator.cpp built with g++ (host
code only, no HIP) and run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_allocator_stress_under_sanitizers(tmp_path):
    exe = tmp_path / "allocator_stress"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "native", "allocator_stress.cpp"),
           os.path.join(ROOT, "paged_kv_cache_210_amd", "csrc", "allocator.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert r.returncode == 0, r.stdout + r.stderr
    assert "allocator stress ok" in r.stdout
