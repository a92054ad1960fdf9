"""Build the gfx950 HIP library in-tree: csrc/*.hip -> libattn.so.

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# Per-file additions.  The prefill kernel has no NaN-dependent logic; without
# this, every fmaxf on a matrix-core result is preceded by a canonicalising
# v_max (32 extra vector instructions per key tile).
FILE_FLAGS = {"prefill_bf16.hip": ["-fno-honor-nans"]}


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source (always; no staleness shortcut) and link."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        cmd = [cc, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        return src, r

    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        results = list(ex.map(compile_one, zip(srcs, objs)))
    errors = []
    for src, r in results:
        if verbose and (r.stdout or r.stderr):
            print(r.stdout + r.stderr)
        if r.returncode != 0:
            errors.append(f"{os.path.basename(src)}:\n{r.stderr}")
    if errors:
        raise RuntimeError("HIP compile failed:\n" + "\n".join(errors))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("HIP link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
