"""The page allocator's host code under AddressSanitizer and UBSan: a
randomized driver (tests/native/pool_fuzz.cpp) linked with page_pool.cpp,
built with g++ (host only, no GPU code) and run; any memory or
undefined-behaviour finding fails it."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_allocator_is_clean_under_sanitizers(tmp_path):
    exe = tmp_path / "pool_fuzz"
    build = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
             os.path.join(ROOT, "tests", "native", "pool_fuzz.cpp"),
             os.path.join(ROOT, "paged_kv_attention_attn_amd", "csrc", "page_pool.cpp"), "-o", str(exe)]
    subprocess.run(build, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("ok:"), run.stdout
