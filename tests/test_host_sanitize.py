"""The library's host core (configuration checks, derived sizes, argument checks,
error text) built with g++ alone under AddressSanitizer and
UndefinedBehaviorSanitizer, and run through every validation case of the C ABI
(tests/host_sanitize_main.cpp).  No GPU and no HIP: the host core has none."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_core_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    srcs = [os.path.join(ROOT, "tests", "host_sanitize_main.cpp"),
            os.path.join(ROOT, "kv_cache_compression_hkv_amd", "csrc", "hkv_host.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Werror",
           "-pthread", "-o", exe, *srcs]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # (a preloaded library ahead of the sanitizer runtime is tolerated)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "passed under the sanitizers" in r.stdout
