"""Compile the SeKV HIP library for gfx950: one shared object, libsekv.so,
next to this file.  Run ``python -m compressed_kv_attention_sekv_amd.build``."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsekv.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["sekv_api.cpp", "sekv_build.hip", "sekv_decode.hip", "sekv_cap.hip",
           "sekv_resident.hip", "sekv_gates.hip", "sekv_rsvd.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # packed fp32 instructions stay off (hipcc's host pass warns it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-result",
]


def _jobs() -> int:
    n = os.environ.get("MAX_JOBS")
    return max(1, min(len(SOURCES), int(n) if n and n.isdigit() else (os.cpu_count() or 1)))


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel, one hipcc per file) and link."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD_DIR, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmds.append([HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)

    def compile_one(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        for f in [ex.submit(compile_one, c) for c in cmds]:
            f.result()
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
