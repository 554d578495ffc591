"""Compile libkda (the HIP kernels and the C-ABI) in-tree for gfx950.

``python -m linear_attention_07_amd.build`` or ``build()`` runs hipcc every
time it is called and writes ``linear_attention_07_amd/lib/libkda.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "lib", "libkda.so")
SOURCES = ["kda_api.hip", "kda_decode.hip", "kda_chunk.hip", "kda_chunk16.hip", "kda_backward.hip",
           "kda_chunk_bwd.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    "-fvisibility=hidden",
    "-mcode-object-version=5",
    # hipcc's own -O3 forms packed fp32 ops from plain float code; keep them off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


ASAN_DIR = os.path.join(PKG, "lib", "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libkda.so")
ASAN_CHECK = os.path.join(ASAN_DIR, "kda_abi_check")
ASAN_CHECK_SRC = os.path.join(ROOT, "tests", "abi_asan", "kda_abi_check.cpp")
# the host code under AddressSanitizer (device code is compiled as always)
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_asan(verbose: bool = False) -> str:
    """The library with its host code under AddressSanitizer, and the host
    program that drives its C-ABI validation paths (tests/abi_asan), in
    linear_attention_07_amd/lib/asan.  Returns the program's path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(ASAN_DIR, exist_ok=True)
    lib_cmd = [hipcc, *HIPCC_FLAGS, *ASAN_HOST_FLAGS,
               *[os.path.join(CSRC, s) for s in SOURCES], "-o", ASAN_LIB]
    exe_cmd = [hipcc, "-O1", "-std=c++17", *ASAN_HOST_FLAGS, "-I", os.path.join(ROOT, "include"),
               ASAN_CHECK_SRC, "-o", ASAN_CHECK, "-L", ASAN_DIR, "-lkda",
               "-Wl,-rpath," + ASAN_DIR]
    noise = "is not a recognized feature for this target"
    for cmd in (lib_cmd, exe_cmd):
        res = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    return ASAN_CHECK


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
