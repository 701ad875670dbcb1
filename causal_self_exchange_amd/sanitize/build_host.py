"""Builds relation_api.cpp with the host compiler's AddressSanitizer and
UndefinedBehaviorSanitizer into a shared library whose device-side functions
are host stubs (every launch fails; nothing here runs on a GPU). The ABI
tests load it in place of librelation.so to check the argument checking for
memory and undefined-behaviour errors.

Usage: python -m causal_self_exchange_amd.sanitize.build_host OUT_DIR
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
CXX = os.environ.get("CXX_HOST", "g++")


def build(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "librelation_host_sanitized.so")
    cmd = [CXX, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fvisibility=hidden", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           os.path.join(PKG, "csrc", "relation_api.cpp"), os.path.join(HERE, "host_stubs.cpp"), "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host sanitizer build failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(PKG, "_build_sanitized")))
