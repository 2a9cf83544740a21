"""The host side of libkata under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

libkata is built once more with the sanitizers on its host code only (each -fsanitize= is
passed with -Xarch_host, so the gfx950 code is built as usual), then
  * the C99 program tests/c/abi_check.c, itself built with the sanitizers, is linked to it
    and run;
  * tests/test_abi_cpu.py runs against it (KATA_LIBRARY) in a Python whose allocator is the
    sanitizer runtime (LD_PRELOAD; leak detection off: the interpreter keeps its objects).
Both exercise argument validation, workspace sizing, status strings and the no-op paths,
with out-of-range sizes and enum values; any sanitizer report fails the test (UBSan halts
on the first error).
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "kernelized_linear_attention_kata_amd", "csrc", "kata.hip")


def _toolchain():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang"
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not (os.path.exists(hipcc) and os.path.exists(clang) and rts):
        pytest.skip("ROCm clang with the sanitizer runtimes not found")
    return hipcc, clang, rts[0]


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    hipcc, clang, rt = _toolchain()
    d = tmp_path_factory.mktemp("asan")
    lib = str(d / "libkata.so")
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan",
           "-I", os.path.join(ROOT, "include"), SRC, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return str(d), lib, clang, rt


def _env(d, rt, **extra):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = f"detect_leaks=0:log_path={d}/asan"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={d}/ubsan"
    env.update(extra)
    return env


def _reports(d):
    out = []
    for f in glob.glob(os.path.join(d, "asan*")) + glob.glob(os.path.join(d, "ubsan*")):
        out.append(open(f).read())
    return out


def test_c_program_under_sanitizers(sanitized):
    d, lib, clang, rt = sanitized
    exe = os.path.join(d, "abi_check")
    cmd = [clang, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-shared-libsan", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", d, "-lkata", "-Wl,-rpath," + d,
           "-Wl,-rpath," + os.path.dirname(rt), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = _env(d, rt, ASAN_OPTIONS=f"detect_leaks=1:log_path={d}/asan")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr
    assert _reports(d) == []


def test_python_abi_tests_under_sanitizers(sanitized):
    d, lib, clang, rt = sanitized
    env = _env(d, rt, LD_PRELOAD=rt, KATA_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert _reports(d) == [], _reports(d)[0][:3000]
