"""Build the native C-ABI client check (test infrastructure, not the product).

chunk_loop.cpp drives the library's chunk loop from C++ and compares with the
C oracle; it is linked against both shared libraries (found through rpath)
into libchunk_loop_check.so, which the GPU test loads with ctypes.  Built
ahead of time by the repository's build entry point, never inside a test.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "chunked_prefill_causal_rope_amd")
ORACLE = os.path.join(ROOT, "oracle")
LIB = os.path.join(HERE, "libchunk_loop_check.so")


def build(rocm: str = "/opt/rocm") -> str:
    """Compile the host-only source with g++ against the HIP runtime API and
    link it with libattn.so and liboracle.so."""
    tmp = LIB + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
           os.path.join(HERE, "chunk_loop.cpp"),
           "-L", PKG, "-lattn", "-L", ORACLE, "-loracle",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../chunked_prefill_causal_rope_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("native client build failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB
