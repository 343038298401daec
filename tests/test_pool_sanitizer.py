"""The host page pool under AddressSanitizer and UBSan: its source (host C++ only) and a random
driver (tests/pool_fuzz.cpp) are built with g++ and run; any memory error, undefined behaviour or
bookkeeping mismatch fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_pool_under_address_and_ub_sanitizers(tmp_path):
    flags = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"]
    obj = tmp_path / "pool.o"
    exe = tmp_path / "pool_fuzz"
    subprocess.run(["g++", *flags, "-x", "c++", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(ROOT, "paged_kv_cache_pg_amd", "csrc", "pool.hip"),
                    "-o", str(obj)], check=True, timeout=300)
    subprocess.run(["g++", *flags, os.path.join(ROOT, "tests", "pool_fuzz.cpp"), str(obj), "-o", str(exe)],
                   check=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1", "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok"), r.stdout
