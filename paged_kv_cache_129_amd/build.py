"""Build libpagedattn.so in-tree for gfx950.

Every .hip source is compiled by hipcc for gfx950 only; the host-only
allocator is compiled by g++.  Objects go to ``_build/`` (git-ignored), the
shared library next to this file.  ``build()`` always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libpagedattn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

HIP_SOURCES = ["api.hip", "kv_write.hip", "copy_blocks.hip", "decode.hip", "decode_mfma.hip",
               "prefill_mfma.hip", "decode_group.hip"]
HOST_SOURCES = ["allocator.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-ffp-contract=fast",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
GXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append(([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        jobs.append((["g++", *GXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for _, o in jobs]])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
