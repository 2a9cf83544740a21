"""The C boundary from C: compile tests/c/abi_check.c as C99 against include/kata.h
(warnings as errors), link it to the built libkata.so and run its host-side checks (no
GPU calls)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "kernelized_linear_attention_kata_amd")


def test_header_compiles_as_c_and_links(tmp_path):
    if not os.path.exists(os.path.join(LIB_DIR, "libkata.so")):
        pytest.skip("libkata.so not built (python -m kernelized_linear_attention_kata_amd.build)")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "abi_check")
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", LIB_DIR, "-lkata", "-Wl,-rpath," + LIB_DIR,
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
