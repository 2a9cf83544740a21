"""Build libkata.so (HIP, gfx950) in-tree with hipcc.

    python -m kernelized_linear_attention_kata_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRC = os.path.join(PKG_DIR, "csrc", "kata.hip")
OUT = os.path.join(PKG_DIR, "libkata.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from emitting packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: a ROCm toolchain is needed to build libkata.so")


def build(verbose: bool = False) -> str:
    """Compile csrc/kata.hip into libkata.so next to this file; returns its path."""
    tmp = OUT + ".tmp"
    cmd = [hipcc_path(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
