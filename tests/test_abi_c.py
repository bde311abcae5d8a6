"""The C ABI from plain C99: tests/native/abi_c.c is compiled with gcc
against include/pkv.h (strict C99, warnings as errors) and linked to the
built libpkv.so, then run; it makes host-side calls only (no GPU)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_kv_attention_attn_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_uses_the_abi(tmp_path):
    if not os.path.exists(os.path.join(PKG, "libpkv.so")):
        pytest.skip("libpkv.so is not built")
    exe = tmp_path / "abi_c"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "native", "abi_c.c"), "-L", PKG, "-lpkv",
                    "-Wl,-rpath," + PKG, "-o", str(exe)], check=True, capture_output=True, timeout=120)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.strip() == "ok"
